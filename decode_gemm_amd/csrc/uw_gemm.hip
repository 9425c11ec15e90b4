// Reconstructive GEMM family for gfx950: Y[M][N] = X[M][K] * W[N][K]^T, fp32 accumulate,
// with W read from one of three planes (bf16 weights, exponent plane + sign/mantissa
// plane, 4-bit palette-index plane + sign/mantissa plane + raw groups). This is the
// "reconstructive matmul" of the Unweight blog post ("How the reconstructive matmul
// works"): compressed data comes in from HBM, bf16 weights are rebuilt on chip and fed
// to the matrix units, and the rebuilt weights are never written back to memory.
//
// The post's kernel is an H100 design (TMA producer / WGMMA consumer warp groups over a
// ~227 KB shared-memory ring). On gfx950 the same job is done by two kernel shapes:
//
//  * skinny (M <= 64, HBM-bound): every wave streams 16-row slices of W one 64-weight
//    group at a time with 16-byte loads and rebuilds the weights directly in the
//    registers that form the A operand of v_mfma_f32_16x16x32_bf16. Within an MFMA the
//    assignment of k to (lane group, register slot) only has to agree between A and B,
//    so each lane owns 16 consecutive k of one row: its sign/mantissa bytes, index
//    nibbles and activations are each one contiguous load, with no shuffles. The waves of
//    a workgroup split K and are reduced through LDS, so no atomics are needed.
//
//  * tiled (larger M, MFMA-bound): a BN x BM output tile per workgroup, K in 64-wide
//    steps (one raw-group decision per row and step). Each step's compressed W slice is
//    rebuilt once into an LDS buffer laid out in MFMA operand order (so operand reads are
//    contiguous 16-byte LDS reads) and shared by all waves; X slices are staged the same
//    way. Two LDS stages: the next step's global loads are in flight while the current
//    one is multiplied. Workgroups are mapped to tiles XCD-first and in groups, so the
//    workgroups that share W and X slices run on the same XCD and hit its L2.
#include <hip/hip_runtime.h>

#include <cstring>
#include <utility>

#include "uw_internal.h"
#include "uw_recon.h"

namespace uw {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const uint16_t* x;
    const uint8_t* sm;
    const void* wplane;
    const uint32_t* bitmap;
    const uint32_t* row_base;
    const uint8_t* raw;
    float* y;
    int64_t ldx, ldy, M, N, K;
    uint32_t words, raw_max;
    uint32_t pal[4];   // palette (rank order) for the index plane
    uint32_t vpal[4];  // palette sorted by value, for the direct plane
    uint32_t base4;    // smallest palette exponent * 0x01010101 (direct plane, contiguous palette)
    const uint8_t* dmeta;  // direct plane: per (tile, group) raw mask and side-table base
    const uint8_t* dside;  // direct plane: raw exponents, 64 bytes per raw (row, group)
    uint32_t tiles;        // direct plane: ceil(N / 16)
    uint32_t kgroups;      // K split: 64-groups per K slice (blockIdx.y), partial sums added into a zeroed Y; 0 = all
    uint16_t* hout;        // SwiGLU epilogue (one K slice only): Y holds the gate projection's output and is
    int64_t ldh;           // only read; the tile's result u goes out as hout[m][n] = bf16(silu(Y[m][n]) u)
};

__device__ __forceinline__ floatx4 mfma16(const u32x4& a, const u32x4& b, const floatx4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// s_waitcnt that waits for LDS reads only (lgkmcnt 0; vmcnt and expcnt at their maxima).
constexpr int kWaitLgkm0 = 0xC07F;

// LDS byte offset of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_offset(const void* p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// One LDS DMA of 16 bytes per lane: lane l's bytes at base + voff go to LDS at lds + 16 l.
// Issued from asm so that the compiler's wait counting does not make every later LDS read
// wait for the newest transfer; the compiler then undercounts outstanding loads, which
// only ever makes its own waits stricter. Callers order the reads of the target
// themselves (a wait for a load issued after the transfer).
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(base)
                 : "memory");
}

// Rank of raw group j among the raw groups of row `row` (the row's bitmap words before
// j's word are popcounted; only reached for raw groups).
__device__ __forceinline__ uint32_t raw_index(const GemmArgs& a, int64_t row, uint32_t j, uint32_t bw)
{
    uint32_t before = __popc(bw & ((1u << (j & 31)) - 1u));
    for (uint32_t t = 0; t < (j >> 5); t++) before += __popc(a.bitmap[row * a.words + t]);
    const uint32_t ri = a.row_base[row] + before;
    return ri < a.raw_max ? ri : a.raw_max;
}

// ------------------------------------------------------------------------- loaders
// The unit of work of both kernels: 16 consecutive weights W[row][k0 .. k0+15] (k0 a
// multiple of 16 inside 64-group j) -> two 8-weight MFMA operand pieces. Per-lane base
// pointers are set up once per row; a group's data then sits at a fixed stride.
//   bf16:   32 B of weights                          (stride 128 B per group)
//   exp:    16 B sign/mantissa + 16 B exponents       (64 + 64)
//   idx:    16 B sign/mantissa + 8 B nibbles           (64 + 32)
//   direct: 16 B sm' + 8 B nibbles of the (tile, group) block (stride 1536 T between
//           groups: blocks are group-major), so a wave's loads are 1 KB and 512 B
//           contiguous
struct W16 {
    u32x4 a, b;
};

template <int SRC>
struct Plane {
    static constexpr int S0 = SRC == UW_W_BF16 ? 128 : SRC == UW_W_DIRECT ? 1536 : 64;
    static constexpr int S1 = SRC == UW_W_BF16 ? 128 : SRC == UW_W_IDX ? 32 : SRC == UW_W_DIRECT ? 1536 : 64;
    const uint8_t* p0;
    const uint8_t* p1;
    int64_t s0 = S0, s1 = S1;  // bytes between consecutive groups

    Plane() = default;
    // lane's pointers for weights [row][16*g ..] of group 0
    __device__ __forceinline__ Plane(const GemmArgs& a, int64_t row, int g)
    {
        const int64_t G = a.K >> 6;
        if (SRC == UW_W_BF16) {
            p0 = static_cast<const uint8_t*>(a.wplane) + 2 * (row * a.K + 16 * g);
            p1 = p0;
        } else if (SRC == UW_W_EXP) {
            p0 = a.sm + row * a.K + 16 * g;
            p1 = static_cast<const uint8_t*>(a.wplane) + row * a.K + 16 * g;
        } else if (SRC == UW_W_IDX) {
            p0 = a.sm + row * a.K + 16 * g;
            p1 = static_cast<const uint8_t*>(a.wplane) + (row * a.K + 16 * g) / 2;
        } else {
            // group-major blocks: rows past N exist (zero) up to the last tile
            (void)G;
            int64_t t = row >> 4;
            t = t < static_cast<int64_t>(a.tiles) ? t : a.tiles - 1;
            const int64_t l = 16 * g + (row & 15);
            p0 = static_cast<const uint8_t*>(a.wplane) + 1536 * t + 16 * l;
            p1 = static_cast<const uint8_t*>(a.wplane) + 1536 * t + 1024 + 8 * l;
            s0 = s1 = 1536 * static_cast<int64_t>(a.tiles);
        }
    }

    __device__ __forceinline__ void load(uint32_t j, W16& w) const
    {
        w.a = *reinterpret_cast<const u32x4*>(p0 + (SRC == UW_W_DIRECT ? s0 : static_cast<int64_t>(S0)) * j);
        if (SRC == UW_W_BF16 || SRC == UW_W_EXP) {
            w.b = *reinterpret_cast<const u32x4*>(p1 + static_cast<int64_t>(S1) * j + (SRC == UW_W_BF16 ? 16 : 0));
        } else {
            const u32x2 v = *reinterpret_cast<const u32x2*>(p1 + (SRC == UW_W_DIRECT ? s1 : static_cast<int64_t>(S1)) * j);
            w.b.x = v.x;
            w.b.y = v.y;
        }
    }
};

// The same loads for a wave whose rows all lie in one 16-row tile (the skinny kernel):
// a wave-uniform base (held in SGPRs and advanced with scalar adds) plus a fixed 32-bit
// lane offset, so a load costs no vector address arithmetic.
template <int SRC>
struct PlaneS {
    static constexpr int S0 = Plane<SRC>::S0, S1 = Plane<SRC>::S1;
    const uint8_t* b0;
    const uint8_t* b1;
    uint32_t o0, o1;
    int64_t s0 = S0;  // direct: bytes between consecutive groups (1536 T)

    PlaneS() = default;
    // tile rows [r0, r0 + 16) (r0 wave-uniform), this lane's row r0 + r, weights 16g ..
    __device__ __forceinline__ PlaneS(const GemmArgs& a, int64_t r0, int r, int g)
    {
        if (SRC == UW_W_DIRECT) {
            int64_t t = r0 >> 4;
            t = t < static_cast<int64_t>(a.tiles) ? t : a.tiles - 1;
            b0 = static_cast<const uint8_t*>(a.wplane) + 1536 * t;
            b1 = b0;
            s0 = 1536 * static_cast<int64_t>(a.tiles);
            const uint32_t l = 16 * g + r;
            o0 = 16 * l;
            o1 = 1024 + 8 * l;
        } else {
            // rows past N read row N - 1 (their outputs are never stored)
            const int64_t rc0 = r0 < a.N ? r0 : a.N - 1;
            const int64_t row = r0 + r < a.N ? r0 + r : a.N - 1;
            const uint32_t e = static_cast<uint32_t>((row - rc0) * a.K + 16 * g);  // element offset
            if (SRC == UW_W_BF16) {
                b0 = static_cast<const uint8_t*>(a.wplane) + 2 * rc0 * a.K;
                b1 = b0 + 16;
                o0 = o1 = 2 * e;
            } else if (SRC == UW_W_EXP) {
                b0 = a.sm + rc0 * a.K;
                b1 = static_cast<const uint8_t*>(a.wplane) + rc0 * a.K;
                o0 = o1 = e;
            } else {
                b0 = a.sm + rc0 * a.K;
                b1 = static_cast<const uint8_t*>(a.wplane) + rc0 * a.K / 2;
                o0 = e;
                o1 = e / 2;
            }
        }
    }

    __device__ __forceinline__ void load(uint32_t j, W16& w) const
    {
        w.a = *reinterpret_cast<const u32x4*>(b0 + (SRC == UW_W_DIRECT ? s0 : static_cast<int64_t>(S0)) * j + o0);
        const uint8_t* q = b1 + (SRC == UW_W_DIRECT ? s0 : static_cast<int64_t>(S1)) * j + o1;
        if (SRC == UW_W_BF16 || SRC == UW_W_EXP) {
            w.b = *reinterpret_cast<const u32x4*>(q);
        } else {
            const u32x2 v = *reinterpret_cast<const u32x2*>(q);
            w.b.x = v.x;
            w.b.y = v.y;
        }
    }
};

// Verbatim exponents of a raw group (16 of them, from k0 & 63), natural order.
__device__ __forceinline__ u32x4 raw_exps16(const GemmArgs& a, int64_t row, int64_t k0, uint32_t j, uint32_t bw)
{
    const uint32_t ri = raw_index(a, row, j, bw);
    return *reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64 + (k0 & 63));
}

// Rebuild the 16 weights of a W16 as two operand pieces. Raw groups are not handled
// here: the index plane holds index 0 there (the weight comes out as sign, palette[0],
// mantissa), the direct plane index 0 (smallest palette exponent); the kernels substitute
// or correct those weights separately.
template <int SRC, bool CONTIG>
__device__ __forceinline__ void rebuild16(const GemmArgs& a, const W16& w, u32x4& p0, u32x4& p1)
{
    if (SRC == UW_W_BF16) {
        p0 = w.a;
        p1 = w.b;
    } else if (SRC == UW_W_EXP) {
        uint32_t ea, eb;
        split_exps(w.b.x, w.b.y, ea, eb);
        p0 = piece_from_split(ea, eb, w.a.x, w.a.y);
        split_exps(w.b.z, w.b.w, ea, eb);
        p1 = piece_from_split(ea, eb, w.a.z, w.a.w);
    } else if (SRC == UW_W_IDX) {
        uint32_t ea, eb;
        exps_from_idx(w.b.x, a.pal, ea, eb);
        p0 = piece_from_split(ea, eb, w.a.x, w.a.y);
        exps_from_idx(w.b.y, a.pal, ea, eb);
        p1 = piece_from_split(ea, eb, w.a.z, w.a.w);
    } else {
        uint32_t e0, e1;
        unit_exps<CONTIG>(w.b.x, a.base4, a.vpal, e0, e1);
        p0 = unit_piece(e0, e1, w.a.x, w.a.y);
        unit_exps<CONTIG>(w.b.y, a.base4, a.vpal, e0, e1);
        p1 = unit_piece(e0, e1, w.a.z, w.a.w);
    }
}

// Direct plane, raw row: the block kept its sign/mantissa bytes; take the 16 verbatim
// exponents (natural order) instead of the palette.
__device__ __forceinline__ void rebuild16_raw(const W16& w, const u32x4& ex, u32x4& p0, u32x4& p1)
{
    p0 = unit_piece(ex.x, ex.y, w.a.x, w.a.y);
    p1 = unit_piece(ex.z, ex.w, w.a.z, w.a.w);
}

// Side-table address of this lane's 16 raw exponents for a block with meta (mask, base),
// or `dummy` (any readable 16 bytes) when its row is not raw there. The index is clamped
// to the last side-table entry, so a corrupt meta word cannot move the read outside the
// plane (with no raw group at all, dside points at the meta section, which is readable).
__device__ __forceinline__ const u32x4* raw_exp_addr(const GemmArgs& a, u32x2 meta, int r, int g, const uint8_t* dummy)
{
    const bool raw = (meta.x >> r) & 1u;
    uint32_t ri = meta.y + __popc(meta.x & ((1u << r) - 1u));
    ri = ri < a.raw_max ? ri : a.raw_max;
    return reinterpret_cast<const u32x4*>(raw ? a.dside + static_cast<uint64_t>(ri) * 64 + 16 * g : dummy);
}

// Operand pieces for the exact correction of raw group j of `row`, for the 16 weights
// [16g, 16g+16) of the group: T = the true weights (blob sign/mantissa + verbatim
// exponents), U = minus what rebuild16 produced for them. MFMA(T) + MFMA(U) adds
// (true - rebuilt) * X exactly; both are bf16 values, so nothing is rounded here.
template <int SRC>
__device__ __forceinline__ void raw_pieces(const GemmArgs& a, int64_t row, uint32_t j, uint32_t ri, int g, u32x4& t0,
                                           u32x4& t1, u32x4& u0, u32x4& u1)
{
    // index plane: T = the true weights (blob sign/mantissa + verbatim exponents), U = minus
    // what rebuild16 produced for them, (sign, palette[0], mantissa) -> flip the signs.
    // MFMA(T) + MFMA(U) adds (true - rebuilt) * X exactly: both are bf16 values.
    const int64_t off = row * a.K + 64 * static_cast<int64_t>(j) + 16 * g;
    ri = ri < a.raw_max ? ri : a.raw_max;  // a corrupt row_base / bitmap stays inside the raw table
    const u32x4 sm = *reinterpret_cast<const u32x4*>(a.sm + off);
    const u32x4 ex = *reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64 + 16 * g);
    uint32_t ea, eb;
    split_exps(ex.x, ex.y, ea, eb);
    t0 = piece_from_split(ea, eb, sm.x, sm.y);
    split_exps(ex.z, ex.w, ea, eb);
    t1 = piece_from_split(ea, eb, sm.z, sm.w);
    const uint32_t p0 = (a.pal[0] & 0xFFu) * 0x01010101u;
    u0 = piece_from_split(p0, p0, sm.x ^ 0x80808080u, sm.y ^ 0x80808080u);
    u1 = piece_from_split(p0, p0, sm.z ^ 0x80808080u, sm.w ^ 0x80808080u);
}

// ------------------------------------------------------------------------- skinny
// Block = NW waves covering rows [16*RT*blockIdx.x, +16*RT) and all of K; wave w takes
// the 64-groups j = w, w + NW, w + 2NW, ... so the block walks its rows front to back.
// Each lane owns 16 consecutive k of one row (the MFMA A operand) and keeps a ring of U
// groups in flight: the compressed W of group t+U and its X operand pieces are requested
// as soon as group t has been consumed, so ~U groups per wave stay outstanding -- at
// 8 TB/s a whole gate matrix is only a few memory latencies long. Vector loads retire in
// issue order, so X travels with the same lead as W; all control flow in the loop is
// wave-uniform, so the compiler waits for exactly the slot it consumes. Lanes of columns
// m >= M read row M-1 (their outputs are never stored). CT = ceil(M / 16).
//
// Raw groups. Direct plane: each slot also carries its blocks' metas (raw-row mask,
// side-table base; requested with the slot, a full ring turn ahead) and, half a turn
// ahead, one load that brings the verbatim exponents of the first raw rows of all its
// row tiles at once (lane 16i + 4k + p: raw row k of tile i, piece p, for RT = 4); a
// lane of a raw row fetches its piece from there with a cross-lane read and substitutes
// it in the rebuild. Every vector load in the loop costs address and data-return cycles
// whatever it carries, and most blocks have no raw row, so one load per group instead of
// one per row tile. Rows past those a slot covers are read directly (rare). Index
// plane: the rebuild yields (sign, palette[0], mantissa) for raw groups and the exact
// difference to the true weights is added after the loop with extra MFMAs, from
// metadata fetched when the kernel starts.
// The block's tile: everything up to its reduced outputs, which go to sink(o, n, m, y) for
// each Y element (o = the element's index in the block tile) inside [0, N) x [0, M).
// red: the block's LDS (the cross-wave reduction, and the X tiles with XT).
// PAIR: a and a1 are the gate and up projections of one SwiGLU MLP (same shape, same X).
// PAIR 1: the wave's steps run over a's groups and then a1's with one ring, so a1's first
// groups are in flight while the block reduces a's outputs into sink (after a's last group;
// every wave takes part once, also one with no group) and restarts its accumulators; a1's
// outputs go to sink1 at the end. PAIR 2: every step takes group j of both (2 RT row tiles
// per slot: a's, then a1's), so each X group is fetched once for both matrices; at the end
// each output element goes to sink (a's value) and then sink1 (a1's), in one thread.
template <int SRC, bool CONTIG, int CT, int RT, int U, int NW, bool XNEAR, int XT, int PAIR, class Sink, class Sink1>
__device__ __forceinline__ void skinny_tile(const GemmArgs& a, const GemmArgs& a1, float* red, Sink&& sink,
                                            Sink1&& sink1)
{
    static_assert(U % 2 == 0, "ring depth must be even");
    static_assert(!(XNEAR && XT), "one X scheme");
    constexpr bool DIRECT = SRC == UW_W_DIRECT;
    constexpr bool POSTRAW = SRC == UW_W_IDX;
    static_assert(!(PAIR && POSTRAW), "pairs of direct planes only");
    constexpr bool SEQ = PAIR == 1, IL = PAIR == 2;
    constexpr int RTT = IL ? 2 * RT : RT;  // row tiles per ring slot
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t nb = static_cast<int64_t>(blockIdx.x) * (16 * RT);
    const uint32_t G = static_cast<uint32_t>(a.K >> 6);
    // K slice of this block (blockIdx.y; all of K unless the launch splits K): groups [j0, j0 + Gs)
    const uint32_t kgs = a.kgroups ? a.kgroups : G;
    const uint32_t j0 = blockIdx.y * kgs;
    const uint32_t Gs = (j0 + kgs < G ? j0 + kgs : G) - j0;
    const uint32_t T = Gs > static_cast<uint32_t>(wave) ? (Gs - wave + NW - 1) / NW : 0;  // groups of this wave
    const uint32_t T2 = SEQ ? 2 * T : T;                                                     // its steps
    // step k of the wave: a1's group k - T for PAIR 1 steps k >= T, else group k
    const auto second = [&](uint32_t k) __attribute__((always_inline)) { return SEQ && k >= T; };
    const auto jc = [&](uint32_t k) __attribute__((always_inline)) {  // the step's group (clamped to the last step)
        k = k < T2 ? k : T2 - 1;
        return j0 + wave + NW * (second(k) ? k - T : k);
    };
    const auto pick = [&](uint32_t k) __attribute__((always_inline)) -> const GemmArgs& { return second(k) ? a1 : a; };

    floatx4 acc[RTT][CT];
#pragma unroll
    for (int i = 0; i < RTT; i++)
#pragma unroll
        for (int c = 0; c < CT; c++) acc[i][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    PlaneS<SRC> pl[RT], pl1[PAIR ? RT : 1];
#pragma unroll
    for (int i = 0; i < RT; i++) pl[i] = PlaneS<SRC>(a, nb + 16 * i, r, g);
    if (PAIR) {
#pragma unroll
        for (int i = 0; i < RT; i++) pl1[PAIR ? i : 0] = PlaneS<SRC>(a1, nb + 16 * i, r, g);
    }
    // direct plane: the lanes LPT i .. LPT i + LPT - 1 fetch the meta (raw-row mask, side
    // base) of row tile i, so a slot's metas are one vector load, retired in order with the
    // slot's other loads (scalar loads may return out of order and would have to be waited
    // for at once), and each lane holds the meta of the tile whose raw exponents it fetches
    // (PAIR 2: lanes past LPT RT hold a1's tiles, with a1's metas and side table)
    constexpr int LPT = 64 / RTT, RAWK = LPT / 4;
    int64_t moff = 0;  // this lane's tile's row of metas (tile-major: consecutive groups adjacent)
    const bool lane2nd = IL && lane / LPT >= RT;
    if (DIRECT) {
        int64_t t = (nb >> 4) + lane / LPT - (lane2nd ? RT : 0);
        t = t < static_cast<int64_t>(a.tiles) ? t : a.tiles - 1;
        moff = 8 * t * G;
    }
    const uint8_t* const lmeta = lane2nd ? a1.dmeta : a.dmeta;
    const uint8_t* const lside = lane2nd ? a1.dside : a.dside;
    const uint32_t lraw_max = lane2nd ? a1.raw_max : a.raw_max;
    // X: uniform base a.x + 64 j, lane offset of row min(16c + r, M - 1), k 16g (bytes;
    // the host keeps 2 * M * ldx below 2^32 for this kernel)
    uint32_t xoff[CT];
#pragma unroll
    for (int c = 0; c < CT; c++) {
        const int64_t m = 16 * c + r;
        xoff[c] = static_cast<uint32_t>(2 * ((m < a.M ? m : a.M - 1) * a.ldx + 16 * g));
    }
    // XT: X is read as whole 128-byte row segments instead (load q: rows 8q .. 8q+7 of the
    // group, lane l = row 8q + l / 8, 16 bytes l % 8) and put into operand order through a
    // wave-private LDS tile, rows 144 bytes apart so the fragment reads hit distinct banks.
    // A fragment load otherwise touches 16 rows at 64 bytes each and costs the address
    // unit twice the lines per byte.
    constexpr int XS_PITCH = 9;  // 16-byte units per LDS row
    uint32_t xofft[XT ? 2 * CT : 1];
    if (XT) {
#pragma unroll
        for (int q = 0; q < 2 * CT; q++) {
            const int64_t m = 8 * q + (lane >> 3);
            xofft[q] = static_cast<uint32_t>(2 * ((m < a.M ? m : a.M - 1) * a.ldx + 8 * (lane & 7)));
        }
    }
    u32x4* const xs = reinterpret_cast<u32x4*>(red) + wave * (16 * CT * XS_PITCH);
    const uint8_t* const xb = reinterpret_cast<const uint8_t*>(a.x);
    // XT 2: the same row segments, but sent by LDS DMA straight into a wave-private ring of U
    // tiles (16 CT rows x 128 bytes each). Load q fills rows 8q .. 8q+7; lane l fetches the
    // 16 bytes of row rho = 8q + l/8 that go to position l % 8, chunk (l % 8) ^ ((rho / 2) % 8),
    // so the 8 lanes of a row still read its whole segment, and a fragment read (row 16c + r,
    // chunk 2g + s2, found at position (2g + s2) ^ (r / 2)) hits 16 distinct bank groups
    // per 16 lanes. No register holds X on the way.
    uint8_t* const xd = reinterpret_cast<uint8_t*>(red) + wave * (U * CT * 2048);
    uint32_t xofd[XT == 2 ? 2 * CT : 1], xfo[2];
    if (XT == 2) {
#pragma unroll
        for (int q = 0; q < 2 * CT; q++) {
            const int rho = 8 * q + (lane >> 3);
            const int64_t m = rho < a.M ? rho : a.M - 1;
            xofd[q] = static_cast<uint32_t>(2 * m * a.ldx + 16 * ((lane & 7) ^ ((rho >> 1) & 7)));
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++) xfo[s2] = static_cast<uint32_t>(128 * r + 16 * ((2 * g + s2) ^ (r >> 1)));
    }
    const uint32_t xd_lds = lds_offset(xd);
    auto dma_x = [&](uint32_t j, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 2 * CT; q++)
            dma16(xb + 128 * static_cast<int64_t>(j), xofd[XT == 2 ? q : 0], xd_lds + (slot * 2 * CT + q) * 1024);
    };

    // Index plane: raw-group metadata of this wave's rows (local rows wave + NW * q),
    // fetched now and consumed after the main loop: lane q holds row_base of row q, and
    // the bitmap words (row q, word wd) sit at flat position q * words + wd across BWV
    // registers. Larger shapes fall back to direct loads after the loop.
    constexpr int RPW = (16 * RT + NW - 1) / NW;  // rows per wave
    constexpr int BWV = 4;
    const uint32_t words = a.words;
    const bool meta_fits = RPW * words <= 64u * BWV;
    uint32_t rbv = 0, bwv[BWV] = {0, 0, 0, 0};
    if (POSTRAW) {
        const int64_t rq = nb + wave + NW * lane;
        if (lane < RPW && rq < a.N) rbv = a.row_base[rq];
        if (meta_fits) {
#pragma unroll
            for (int k = 0; k < BWV; k++) {
                const uint32_t f = lane + 64 * k, q = f / words, wd = f - q * words;
                const int64_t row = nb + wave + NW * static_cast<int64_t>(q);
                if (q < static_cast<uint32_t>(RPW) && row < a.N) bwv[k] = a.bitmap[row * words + wd];
            }
        }
    }

    // X pieces of group j in MFMA operand order (the post-loop raw correction)
    auto load_x_frag = [&](uint32_t j, u32x4 (&B)[CT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < CT; c++) {
            const u32x4* xp = reinterpret_cast<const u32x4*>(xb + 128 * static_cast<int64_t>(j) + xoff[c]);
            B[c][0] = xp[0];
            B[c][1] = xp[1];
        }
    };
    // X of group j for the ring: operand order, or row segments for XT
    auto load_x = [&](uint32_t j, u32x4 (&B)[CT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < CT; c++) {
            if (XT) {
                B[c][0] = *reinterpret_cast<const u32x4*>(xb + 128 * static_cast<int64_t>(j) + xofft[XT ? 2 * c : 0]);
                B[c][1] = *reinterpret_cast<const u32x4*>(xb + 128 * static_cast<int64_t>(j) + xofft[XT ? 2 * c + 1 : 0]);
            } else {
                const u32x4* xp = reinterpret_cast<const u32x4*>(xb + 128 * static_cast<int64_t>(j) + xoff[c]);
                B[c][0] = xp[0];
                B[c][1] = xp[1];
            }
        }
    };
    W16 ring[U][RTT];
    u32x4 xr[XNEAR ? 1 : U][CT][2];
    // direct plane: the slot's metas, and one load of raw exponents per slot: lane
    // LPT i + 4k + p holds piece p of raw row k of tile i (k < RAWK)
    u32x2 mr[DIRECT ? U : 1];
    u32x4 rx[DIRECT ? U : 1];
    // slot u <- step k: its metas, then its W
    auto load_slot = [&](uint32_t k, auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        const uint32_t j = jc(k);
        const bool s2nd = second(k);
        // the meta goes first: it is read half a ring turn later, and waiting for it must
        // not wait for the slot's W loads
        if (DIRECT)
            mr[u % (DIRECT ? U : 1)] =
                *reinterpret_cast<const u32x2*>((IL ? lmeta : s2nd ? a1.dmeta : a.dmeta) + moff + 8 * static_cast<int64_t>(j));
#pragma unroll
        for (int i = 0; i < RTT; i++) {
            PlaneS<SRC> pw = pl[i % RT];
            if ((SEQ && s2nd) || (IL && i >= RT)) {
                pw.b0 = pl1[PAIR ? i % RT : 0].b0;
                pw.b1 = pl1[PAIR ? i % RT : 0].b1;
            }
            pw.load(j, ring[u][i]);
        }
    };
    // the raw exponents of slot v, which holds step ks
    auto load_raw = [&](uint32_t ks, auto vc) __attribute__((always_inline)) {
        constexpr int v = decltype(vc)::value % (DIRECT ? U : 1);
        const GemmArgs& a = pick(ks);
        // every lane holds the meta of its tile; a lane past the tile's raw rows, or of a
        // tile with none, reads the (always readable) meta section instead. The load is
        // always issued, so every wait in the loop stays a counted one.
        const int k = (lane % LPT) >> 2, p4 = lane & 3;
        const uint32_t mx = mr[v].x, my = mr[v].y;
        const uint8_t* const dm = IL ? lmeta : a.dmeta;
        const uint8_t* const ds = IL ? lside : a.dside;
        const uint32_t rmax = IL ? lraw_max : a.raw_max;
        const u32x4* src = reinterpret_cast<const u32x4*>(dm);
        if (static_cast<uint32_t>(k) < static_cast<uint32_t>(__popc(mx))) {
            uint32_t ri = my + k;
            ri = ri < rmax ? ri : rmax;
            src = reinterpret_cast<const u32x4*>(ds + static_cast<uint64_t>(ri) * 64 + 16 * p4);
        }
        rx[v] = *src;
    };
    // cross-wave reduction of acc into snk: red[w][i][c][q][lane]; then output element
    // o = ((tile * 16 + m_local) * 16 + n_local), consecutive threads on consecutive n of one
    // Y row. The caller has made red free (a barrier after any other use of it).
    constexpr int TILES = RTT * CT;
    float* const redp = red + (SEQ && XT == 2 ? (NW * U * CT * 2048) / 4 : 0);  // PAIR 1: past the X rings
    auto reduce_into = [&](const GemmArgs& ar, auto&& snk) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RTT; i++)
#pragma unroll
            for (int c = 0; c < CT; c++)
#pragma unroll
                for (int q = 0; q < 4; q++) redp[((wave * TILES + i * CT + c) * 4 + q) * 64 + lane] = acc[i][c][q];
        __syncthreads();
        for (int o = threadIdx.x; o < TILES * 256; o += 64 * NW) {
            const int tile = o >> 8, ml = (o >> 4) & 15, nl = o & 15;
            const int i = tile / CT, c = tile % CT;
            const int src_lane = (nl >> 2) * 16 + ml, q = nl & 3;
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; w++) sum += redp[((w * TILES + tile) * 4 + q) * 64 + src_lane];
            const int64_t n = nb + 16 * i + nl, m = 16 * c + ml;
            if (n < ar.N && m < ar.M) snk(o, n, m, sum);
        }
    };
    // PAIR 2: both matrices' outputs of an element, a's then a1's (tile i + RT), in one thread
    auto reduce_pair = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RTT; i++)
#pragma unroll
            for (int c = 0; c < CT; c++)
#pragma unroll
                for (int q = 0; q < 4; q++) redp[((wave * TILES + i * CT + c) * 4 + q) * 64 + lane] = acc[i][c][q];
        __syncthreads();
        for (int o = threadIdx.x; o < RT * CT * 256; o += 64 * NW) {
            const int tile = o >> 8, ml = (o >> 4) & 15, nl = o & 15;
            const int i = tile / CT, c = tile % CT;
            const int src_lane = (nl >> 2) * 16 + ml, q = nl & 3;
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int w = 0; w < NW; w++) {
                s0 += redp[((w * TILES + tile) * 4 + q) * 64 + src_lane];
                s1 += redp[((w * TILES + RT * CT + tile) * 4 + q) * 64 + src_lane];
            }
            const int64_t n = nb + 16 * i + nl, m = 16 * c + ml;
            if (n < a.N && m < a.M) {
                sink(o, n, m, s0);
                sink1(o, n, m, s1);
            }
        }
    };
    // PAIR, after a's last group: a's outputs to sink, a fresh start for a1. The X rings stay
    // untouched (they are not in redp), XT 1's tiles alias it: every wave is past its own
    // step first, and past the reads of red before anything writes it again.
    auto mid_reduce = [&]() __attribute__((always_inline)) {
        if (XT == 1) __syncthreads();
        reduce_into(a, sink);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RT; i++)
#pragma unroll
            for (int c = 0; c < CT; c++) acc[i][c] = floatx4{0.f, 0.f, 0.f, 0.f};
    };
    // one group: rebuild ring slot u (group t), refill it with group t + U, request the
    // raw exponents of group t + U/2, multiply, then refill the X pieces
    auto step = [&](uint32_t t, auto uc, bool refill, bool rawpf) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        const GemmArgs& a0 = pick(t);  // (only the consumed matrix's palette and side table)
        u32x4 XF[XT ? CT : 1][2];  // XT: this step's X fragments, back from the LDS tile
        if (XT == 2) {
            // the slot's X transfer was issued before its W loads, and loads retire in
            // order: once the slot's first W register is waited for, its X is in LDS
            asm volatile("" ::"v"(ring[u][0].a.x));
            __builtin_amdgcn_sched_barrier(0);
            const uint8_t* const xs2 = xd + u * (CT * 2048);
#pragma unroll
            for (int c = 0; c < CT; c++)
#pragma unroll
                for (int s2 = 0; s2 < 2; s2++) XF[XT ? c : 0][s2] = *reinterpret_cast<const u32x4*>(xs2 + 2048 * c + xfo[s2]);
        }
        if (XT == 1) {
#pragma unroll
            for (int q = 0; q < 2 * CT; q++) xs[(8 * q + (lane >> 3)) * XS_PITCH + (lane & 7)] = xr[XNEAR ? 0 : u][q >> 1][q & 1];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int c = 0; c < CT; c++)
#pragma unroll
                for (int s2 = 0; s2 < 2; s2++) XF[XT ? c : 0][s2] = xs[(16 * c + r) * XS_PITCH + 2 * g + s2];
            // the slot's X registers are free once stored: refill them first, so the X of
            // group t + U has U whole steps to arrive and is never queued behind W
            if (!XNEAR && refill) load_x(jc(t + U), xr[XNEAR ? 0 : u]);
            __builtin_amdgcn_sched_barrier(0);
        }
        u32x4 A[RTT][2];
#pragma unroll
        for (int i = 0; i < RTT; i++) {
            const GemmArgs& a = IL && i >= RT ? a1 : a0;
            rebuild16<SRC, CONTIG>(a, ring[u][i], A[i][0], A[i][1]);
            if (DIRECT) {
                const uint32_t mask = __builtin_amdgcn_readlane(mr[u % (DIRECT ? U : 1)].x, LPT * i);
                if (mask) {
                    // raw rows in this tile: row r's piece g comes from lane LPT i + 4k + g
                    // (k = its rank among the tile's raw rows), or straight from the side
                    // table past the first RAWK
                    const uint32_t k = __popc(mask & ((1u << r) - 1u));
                    const u32x4 v = rx[u % (DIRECT ? U : 1)];
                    const int sl = 4 * (LPT * i + 4 * static_cast<int>(k < RAWK ? k : 0) + g);
                    u32x4 ex = {static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(sl, v.x)),
                                static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(sl, v.y)),
                                static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(sl, v.z)),
                                static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(sl, v.w))};
                    const bool raw = (mask >> r) & 1u;
                    if (__builtin_expect(__popc(mask) > RAWK, 0) && raw && k >= RAWK) {
                        const u32x2 m = {mask, static_cast<uint32_t>(__builtin_amdgcn_readlane(mr[u % (DIRECT ? U : 1)].y, LPT * i))};
                        ex = *raw_exp_addr(a, m, r, g, a.dmeta);
                    }
                    if (raw) rebuild16_raw(ring[u][i], ex, A[i][0], A[i][1]);
                }
            }
        }
        if constexpr (XNEAR) {
            // X one group ahead, in one register set: multiply, request the next group's X
            // (before the W refill, so waiting for it never waits for that refill), then
            // refill the W slot
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
                for (int i = 0; i < RTT; i++)
#pragma unroll
                    for (int c = 0; c < CT; c++) acc[i][c] = mfma16(A[i][s2], xr[0][c][s2], acc[i][c]);
            if (refill || t + 1 < T2) load_x(jc(t + 1), xr[0]);  // unconditional in the steady state
            if (refill) load_slot(t + U, uc);
            if (DIRECT && rawpf) load_raw(t + U / 2, std::integral_constant<int, (u + U / 2) % U>{});
        } else {
            // issue order is pinned: (XT: the X refill,) the raw exponents consumed half a
            // turn from now, the W slot refill (a full turn ahead), the MFMAs, the X refill;
            // waiting for any of them then never waits for a younger request
            __builtin_amdgcn_sched_barrier(0);
            if (XT == 2 && refill) {
                // the fragment reads of this slot are done before its next X lands there
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                dma_x(jc(t + U), u);
            }
            if (DIRECT && rawpf) load_raw(t + U / 2, std::integral_constant<int, (u + U / 2) % U>{});
            if (refill) load_slot(t + U, uc);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
                for (int i = 0; i < RTT; i++)
#pragma unroll
                    for (int c = 0; c < CT; c++)
                        acc[i][c] = mfma16(A[i][s2], XT ? XF[XT ? c : 0][s2] : xr[u][c][s2], acc[i][c]);
            __builtin_amdgcn_sched_barrier(0);
            if (!XT && refill) load_x(jc(t + U), xr[u]);
        }
        if (SEQ && t + 1 == T) mid_reduce();  // a's last group: its outputs, while a1's first are in flight
    };
    // The ring is filled with no conditions (slots past the wave's last group reload that
    // group): the compiler's wait counts at the loop head are the minimum over every path
    // into it, so a skipped load on any path would make it wait for nearly all loads in
    // flight, once per ring turn.
    if (SEQ && T == 0) mid_reduce();  // (a wave with no group still takes part)
    if (T > 0) {
        [&]<int... us>(std::integer_sequence<int, us...>) {
            if constexpr (XNEAR) {
                (load_slot(us, std::integral_constant<int, us>{}), ...);
                if (DIRECT) ((us < U / 2 ? load_raw(us, std::integral_constant<int, us>{}) : void()), ...);
                load_x(jc(0), xr[0]);  // the slice's first group of this wave
            } else {
                // the steady state's issue order: (XT: slot k's X,) the raw exponents of slot
                // k - U/2, slot k's meta and W, (otherwise: slot k's X)
                auto first = [&](auto kc) __attribute__((always_inline)) {
                    constexpr int k = decltype(kc)::value;
                    // (pinned: the loop head's wait counts are the minimum over this path
                    // and the loop's own, so a reordered prologue would weaken them)
                    __builtin_amdgcn_sched_barrier(0);
                    if (XT == 1) load_x(jc(k), xr[XNEAR ? 0 : k]);
                    if (XT == 2) dma_x(jc(k), k);
                    __builtin_amdgcn_sched_barrier(0);
                    if (DIRECT && k >= U / 2) load_raw(k - U / 2, std::integral_constant<int, (k + U / 2) % U>{});
                    __builtin_amdgcn_sched_barrier(0);
                    load_slot(k, kc);
                    __builtin_amdgcn_sched_barrier(0);
                    if (!XT) load_x(jc(k), xr[XNEAR ? 0 : k]);
                    __builtin_amdgcn_sched_barrier(0);
                };
                (first(std::integral_constant<int, us>{}), ...);
            }
        }(std::make_integer_sequence<int, U>{});
    }
    uint32_t t0 = 0;
    // steady state: every slot is consumed and refilled, no guards, so the compiler waits
    // for exactly the slot it needs
    for (; t0 + 2 * U <= T2; t0 += U) {
        [&]<int... us>(std::integer_sequence<int, us...>) {
            (step(t0 + us, std::integral_constant<int, us>{}, true, true), ...);
        }(std::make_integer_sequence<int, U>{});
    }
    // tail: the last one or two turns of the ring
    for (; t0 < T2; t0 += U) {
        [&]<int... us>(std::integer_sequence<int, us...>) {
            ((t0 + us < T2 ? step(t0 + us, std::integral_constant<int, us>{}, t0 + us + U < T2, t0 + us + U / 2 < T2)
                          : void()),
             ...);
        }(std::make_integer_sequence<int, U>{});
    }

    if (POSTRAW) {
        // raw groups of this wave's rows, corrected exactly with extra MFMAs each
        for (int q = 0; q < RPW; q++) {
            const int li = wave + NW * q;
            const int64_t row = nb + li;
            if (li >= 16 * RT || row >= a.N) break;
            uint32_t ri = __builtin_amdgcn_readlane(rbv, q);
            for (uint32_t wd = 0; wd < words; wd++) {
                uint32_t bits;
                if (meta_fits) {
                    const uint32_t f = q * words + wd, k = f >> 6, l = f & 63;
                    const uint32_t v = k == 0 ? bwv[0] : k == 1 ? bwv[1] : k == 2 ? bwv[2] : bwv[3];
                    bits = __builtin_amdgcn_readlane(v, l);
                } else {
                    bits = __builtin_amdgcn_readfirstlane(a.bitmap[row * words + wd]);
                }
                while (bits) {
                    const uint32_t j = 32 * wd + __builtin_ctz(bits);
                    bits &= bits - 1;
                    if (j < j0 || j >= j0 + Gs) {  // another K slice's group
                        ri++;
                        continue;
                    }
                    u32x4 t0v = {0, 0, 0, 0}, t1v = t0v, u0v = t0v, u1v = t0v;
                    if (r == (li & 15)) raw_pieces<SRC>(a, row, j, ri, g, t0v, t1v, u0v, u1v);
                    ri++;
                    u32x4 B[CT][2];
                    load_x_frag(j, B);
#pragma unroll
                    for (int i = 0; i < RT; i++) {
                        if (i == (li >> 4)) {
#pragma unroll
                            for (int c = 0; c < CT; c++) {
                                acc[i][c] = mfma16(t0v, B[c][0], acc[i][c]);
                                acc[i][c] = mfma16(t1v, B[c][1], acc[i][c]);
                                acc[i][c] = mfma16(u0v, B[c][0], acc[i][c]);
                                acc[i][c] = mfma16(u1v, B[c][1], acc[i][c]);
                            }
                        }
                    }
                }
            }
        }
    }

    // (XT 2: every transfer has landed, those of ring slots past the wave's last group too)
    if (XT == 2) __builtin_amdgcn_s_waitcnt(0);
    if (XT) __syncthreads();
    if constexpr (IL)
        reduce_pair();
    else
        reduce_into(SEQ ? a1 : a, sink1);
}

template <int SRC, bool CONTIG, int CT, int RT, int U, int NW, bool XNEAR, int XT>
__global__ void __launch_bounds__(64 * NW) gemm_skinny(GemmArgs a)
{
    extern __shared__ float red[];
    auto store = [&](int, int64_t n, int64_t m, float v) {
        if (a.kgroups)
            atomicAdd(a.y + m * a.ldy + n, v);  // K split: Y was zeroed, every slice adds its part
        else
            a.y[m * a.ldy + n] = v;
    };
    skinny_tile<SRC, CONTIG, CT, RT, U, NW, XNEAR, XT, 0>(a, a, red, store, store);
}

// LDS of a skinny block: the cross-wave reduction, or the X tiles (aliased): XT 1, one
// padded tile per wave; XT 2, a ring of U DMA targets per wave (PAIR 1: the rings and the
// reduction side by side, as the rings stay in use across the mid-stream reduction; PAIR 2:
// the reduction covers both matrices' tiles).
template <int CT, int RT, int U, int NW, int XT, int PAIR = 0>
constexpr size_t skinny_lds()
{
    constexpr size_t red_bytes = static_cast<size_t>(NW) * (PAIR == 2 ? 2 * RT : RT) * CT * 256 * 4;
    constexpr size_t xt_bytes = XT == 1 ? static_cast<size_t>(NW) * 16 * CT * 9 * 16
                              : XT == 2 ? static_cast<size_t>(NW) * U * CT * 2048
                                        : 0;
    if (PAIR == 1 && XT == 2) return red_bytes + xt_bytes;
    return red_bytes > xt_bytes ? red_bytes : xt_bytes;
}

// gate and up of a SwiGLU MLP in one launch (direct planes, same X, same shape): each
// block streams its rows of gate and up through one ring (group by group, both matrices in
// a step, or gate's groups and then up's: PAIR 2 or 1), keeps gate's outputs in LDS, and
// writes g, u (fp32) and h = bf16(silu(g) * u). One ramp and one tail instead of three
// launches, no separate SwiGLU pass; with PAIR 2 each X group is fetched once for both.
struct GateUpArgs {
    GemmArgs gate, up;
    uint16_t* h;
    int64_t ldh;
    float* zy;  // (or null) a Y that the blocks clear first: zM rows of zN floats, zld apart
    int64_t zld;
    uint32_t zM, zN;
};

template <bool CG, bool CU, int CT, int RT, int U, int NW, bool XNEAR, int XT, int PAIR>
__global__ void __launch_bounds__(64 * NW) gemm_skinny_gate_up(GateUpArgs ga)
{
    static_assert(CG == CU, "one palette kind for both (the launcher takes consecutive exponents only)");
    extern __shared__ float red[];
    if (ga.zy) {
        // the Y of the K-split launch that comes next on the stream, cleared here (16-byte
        // stores; the host checked alignment) instead of by a launch of its own
        const uint32_t n4 = (ga.zN + 3) / 4, units = ga.zM * n4;
        for (uint32_t q = blockIdx.x * blockDim.x + threadIdx.x; q < units; q += gridDim.x * blockDim.x) {
            const uint32_t m = q / n4, n = 4 * (q - m * n4);
            float* row = ga.zy + static_cast<int64_t>(m) * ga.zld + n;
            if (n + 4 <= ga.zN)
                *reinterpret_cast<floatx4*>(row) = floatx4{0.f, 0.f, 0.f, 0.f};
            else
                for (uint32_t c = 0; n + c < ga.zN; c++) row[c] = 0.f;
        }
    }
    float* const gbuf = red + skinny_lds<CT, RT, U, NW, XT, PAIR>() / 4;  // RT * CT * 256 gate outputs
    skinny_tile<UW_W_DIRECT, CG, CT, RT, U, NW, XNEAR, XT, PAIR>(
        ga.gate, ga.up, red,
        [&](int o, int64_t n, int64_t m, float v) {
            ga.gate.y[m * ga.gate.ldy + n] = v;
            gbuf[o] = v;
        },
        [&](int o, int64_t n, int64_t m, float v) {
            ga.up.y[m * ga.up.ldy + n] = v;
            ga.h[m * ga.ldh + n] = static_cast<uint16_t>(f32_to_bf16_rne(silu_mul(gbuf[o], v)));
        });
}

// ------------------------------------------------------------------------- expand
// Direct plane -> bf16 W[N][K] in HBM, for a plain GEMM afterwards (the full-decode
// pipeline's second half, fed from the load-time plane instead of the Huffman stream).
// One wave per (row tile, group) block, lane l = 16 g + r: the 16 weights [16g, 16g+16) of
// row 16 t + r, rebuilt exactly as the GEMMs rebuild them (palette, or the side table's
// verbatim exponents on a raw row), then stored as two 16-byte pieces.
template <bool CONTIG>
__global__ void __launch_bounds__(256) expand_direct_kernel(GemmArgs a, uint16_t* w)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t G = static_cast<uint64_t>(a.K >> 6);
    const uint64_t blk = static_cast<uint64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // j * T + t
    if (blk >= static_cast<uint64_t>(a.tiles) * G) return;
    const uint64_t j = blk / a.tiles, t = blk - j * a.tiles;
    const uint8_t* b = static_cast<const uint8_t*>(a.wplane) + 1536 * blk;
    W16 wv;
    wv.a = *reinterpret_cast<const u32x4*>(b + 16 * lane);
    const u32x2 v = *reinterpret_cast<const u32x2*>(b + 1024 + 8 * lane);
    wv.b.x = v.x;
    wv.b.y = v.y;
    wv.b.z = 0;
    wv.b.w = 0;
    const u32x2 meta = *reinterpret_cast<const u32x2*>(a.dmeta + 8 * (t * G + j));
    const int r = static_cast<int>(lane & 15), g = static_cast<int>(lane >> 4);
    u32x4 p0, p1;
    rebuild16<UW_W_DIRECT, CONTIG>(a, wv, p0, p1);
    if ((meta.x >> r) & 1u) rebuild16_raw(wv, *raw_exp_addr(a, meta, r, g, a.dmeta), p0, p1);
    const int64_t row = static_cast<int64_t>(16 * t) + r;
    if (row < a.N) {
        u32x4* o = reinterpret_cast<u32x4*>(w + row * a.K + static_cast<int64_t>(64 * j) + 16 * g);
        o[0] = p0;
        o[1] = p1;
    }
}

// ------------------------------------------------------------------------- tiled
// 256 threads = 4 waves as 2 x 2; block tile BN (weight rows) x BM (activation rows);
// wave tile (BN/2) x (BM/2) of 16 x 16 MFMA tiles. LDS per stage: W and X slices of 64 k
// in operand order: [16-row tile][k-half][lane][8 values].
// K slice of this block (tiled and wide kernels): 64-groups [j0, j1).
__device__ __forceinline__ void k_slice(const GemmArgs& a, uint32_t G, uint32_t& j0, uint32_t& j1)
{
    const uint32_t kg = a.kgroups ? a.kgroups : G;
    j0 = blockIdx.y * kg;
    j1 = j0 + kg < G ? j0 + kg : G;
}

// Raw-table index of the first raw group at or after group j0 of a row (index plane).
__device__ __forceinline__ uint32_t raw_base_at(const GemmArgs& a, int64_t row, uint32_t j0)
{
    uint32_t base = a.row_base[row];
    for (uint32_t w = 0; w < (j0 >> 5); w++) base += __popc(a.bitmap[row * a.words + w]);
    return base;
}

// Store 4 consecutive n of output row m.
__device__ __forceinline__ void store_out(const GemmArgs& a, int64_t m, int64_t n, const floatx4& v)
{
    if (m >= a.M) return;
    float* yp = a.y + m * a.ldy + n;
    if (n + 3 < a.N && (a.ldy & 3) == 0) {
        *reinterpret_cast<floatx4*>(yp) = v;
    } else {
        for (int q = 0; q < 4; q++)
            if (n + q < a.N) yp[q] = v[q];
    }
}

// Split-K epilogue of a BN x BM tile held by waves (wn, wm), wave tiles TN x TM of 16x16:
// add it into Y with fp32 atomics, one m half (the rows of the waves with wm = h) at a
// time. The half goes through LDS (free once the K loop is done) so that each atomic
// instruction of a wave covers 64 consecutive floats of one Y row, two cache lines,
// instead of the 16 rows of an MFMA output fragment. Columns are XOR-swizzled by row so
// the fragment writes do not collide on LDS banks.
template <int BN, int BM, int TN, int TM, int NT>
__device__ __forceinline__ void add_tile(const GemmArgs& a, float* ep, const floatx4 (&acc)[TN][TM], int64_t n0,
                                         int64_t m0, int wn, int wm, int lane, int tid)
{
    constexpr int HR = BM / 2;
    static_assert(BN % 64 == 0 && TM * 16 == HR, "tile shape");
#pragma unroll
    for (int h = 0; h < 2; h++) {
        __syncthreads();
        if (wm == h) {
#pragma unroll
            for (int i = 0; i < TN; i++)
#pragma unroll
                for (int c = 0; c < TM; c++) {
                    const int nn = (wn * TN + i) * 16 + 4 * (lane >> 4), mm = c * 16 + (lane & 15);
                    *reinterpret_cast<floatx4*>(ep + mm * BN + (nn ^ ((mm & 15) << 2))) = acc[i][c];
                }
        }
        __syncthreads();
#pragma unroll 8
        for (int e = tid; e < HR * BN; e += NT) {
            const int mm = e / BN, nn = e % BN;
            const int64_t m = m0 + h * HR + mm, n = n0 + nn;
            if (m < a.M && n < a.N) unsafeAtomicAdd(a.y + m * a.ldy + n, ep[mm * BN + (nn ^ ((mm & 15) << 2))]);
        }
    }
}

// SwiGLU epilogue of a BN x BM tile (one K slice, a.hout set): the tile holds the up
// projection's outputs u, Y the gate's; hout[m][n] = bf16(silu(Y[m][n]) u[m][n]). As in
// add_tile, one m half at a time goes through LDS, so that a wave reads one whole Y row
// segment (BN floats) per load instruction instead of 16 rows of an MFMA fragment.
template <int BN, int BM, int TN, int TM, int NT>
__device__ __forceinline__ void swiglu_tile(const GemmArgs& a, float* ep, const floatx4 (&acc)[TN][TM], int64_t n0,
                                            int64_t m0, int wn, int wm, int lane, int tid)
{
    constexpr int HR = BM / 2, Q = BN / 4;
    static_assert(BN % 64 == 0 && TM * 16 == HR, "tile shape");
    const bool vec = (a.ldy & 3) == 0 && (a.ldh & 3) == 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        __syncthreads();
        if (wm == h) {
#pragma unroll
            for (int i = 0; i < TN; i++)
#pragma unroll
                for (int c = 0; c < TM; c++) {
                    const int nn = (wn * TN + i) * 16 + 4 * (lane >> 4), mm = c * 16 + (lane & 15);
                    *reinterpret_cast<floatx4*>(ep + mm * BN + (nn ^ ((mm & 15) << 2))) = acc[i][c];
                }
        }
        __syncthreads();
#pragma unroll 4
        for (int e = tid; e < HR * Q; e += NT) {
            const int mm = e / Q, nn = 4 * (e % Q);
            const int64_t m = m0 + h * HR + mm, n = n0 + nn;
            if (m >= a.M || n >= a.N) continue;
            const floatx4 u4 = *reinterpret_cast<const floatx4*>(ep + mm * BN + (nn ^ ((mm & 15) << 2)));
            const float* gp = a.y + m * a.ldy + n;
            uint16_t* hp = a.hout + m * a.ldh + n;
            if (vec && n + 3 < a.N) {
                const floatx4 g4 = *reinterpret_cast<const floatx4*>(gp);
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; q++) o[q] = f32_to_bf16_rne(silu_mul(g4[q], u4[q]));
                *reinterpret_cast<uint2*>(hp) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
            } else {
                for (int q = 0; q < 4; q++)
                    if (n + q < a.N) hp[q] = static_cast<uint16_t>(f32_to_bf16_rne(silu_mul(gp[q], u4[q])));
            }
        }
    }
}

// Y[0, M) x [0, N) = 0: rows m = blockIdx.y + k gridDim.y, four columns per thread (one
// 16-byte store when ldy keeps the rows 16-byte aligned).
__global__ void __launch_bounds__(256) zero_rows(float* y, int64_t ldy, int64_t M, int64_t N)
{
    const int64_t n = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
    if (n >= N) return;
    const bool vec = (ldy & 3) == 0 && n + 4 <= N;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        float* row = y + m * ldy + n;
        if (vec) {
            *reinterpret_cast<floatx4*>(row) = floatx4{0.f, 0.f, 0.f, 0.f};
        } else {
            for (int64_t q = 0; q < 4 && n + q < N; q++) row[q] = 0.f;
        }
    }
}

hipError_t launch_zero_rows(float* y, int64_t ldy, int64_t M, int64_t N, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>((N + 1023) / 1024), static_cast<uint32_t>(M < 65535 ? M : 65535));
    hipLaunchKernelGGL(zero_rows, grid, dim3(256), 0, s, y, ldy, M, N);
    return hipGetLastError();
}

template <int BN, int BM>
struct TiledCfg {
    static constexpr int TN = BN / 32, TM = BM / 32;     // 16x16 tiles per wave
    static constexpr int WITEMS = (BN * 2 + 255) / 256;  // (row, k-half) items per thread, W
    static constexpr int XITEMS = (BM * 2 + 255) / 256;  // same for X (threads past BM*2 idle)
    static constexpr int A_BYTES = BN * 64 * 2;          // one stage of rebuilt W
    static constexpr int B_BYTES = BM * 64 * 2;
    static constexpr int LDS = 2 * (A_BYTES + B_BYTES);
};

// blockIdx -> (n tile, m tile): consecutive hardware workgroups are dealt round-robin to
// the 8 XCDs, so first regroup them so each XCD gets a contiguous run of logical tiles,
// then walk the tiles in groups of 8 n-tiles so that concurrently resident workgroups
// share W slices (same n tile) and X slices (same m tile) in that XCD's L2.
__device__ __forceinline__ void tile_of_block(uint32_t bid, uint32_t nblocks, uint32_t tiles_n, uint32_t tiles_m,
                                              uint32_t& tn, uint32_t& tm)
{
    constexpr uint32_t XCD = 8, GROUP = 8;
    uint32_t pid = bid;
    const uint32_t full = nblocks / XCD * XCD;
    if (bid < full) pid = (bid % XCD) * (nblocks / XCD) + bid / XCD;
    const uint32_t per_group = GROUP * tiles_m;
    const uint32_t group = pid / per_group;
    const uint32_t first_n = group * GROUP;
    const uint32_t gsize = (tiles_n - first_n) < GROUP ? (tiles_n - first_n) : GROUP;
    const uint32_t in_group = pid % per_group;
    tn = first_n + in_group % gsize;
    tm = in_group / gsize;
}

template <int SRC, bool CONTIG, int BN, int BM>
__global__ void __launch_bounds__(256) gemm_tiled(GemmArgs a)
{
    using C = TiledCfg<BN, BM>;
    constexpr bool RAW = SRC == UW_W_IDX;  // index plane: raw items found from the bitmap
    constexpr bool DIRECT = SRC == UW_W_DIRECT;  // direct plane: raw rows from the block meta
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // stage st of the rebuilt W slice: As + st * A_VEC; of the X slice: Bs + st * B_VEC
    u32x4* const As = reinterpret_cast<u32x4*>(lds);
    u32x4* const Bs = reinterpret_cast<u32x4*>(lds + 2 * C::A_BYTES);
    constexpr int A_VEC = C::A_BYTES / 16, B_VEC = C::B_BYTES / 16;

    const uint32_t tiles_n = static_cast<uint32_t>((a.N + BN - 1) / BN);
    const uint32_t tiles_m = static_cast<uint32_t>((a.M + BM - 1) / BM);
    uint32_t tn, tm;
    tile_of_block(blockIdx.x, gridDim.x, tiles_n, tiles_m, tn, tm);
    const int64_t n0 = static_cast<int64_t>(tn) * BN, m0 = static_cast<int64_t>(tm) * BM;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave >> 1, wm = wave & 1;
    const uint32_t G = static_cast<uint32_t>(a.K >> 6);
    uint32_t j0, j1;
    k_slice(a, G, j0, j1);

    // item t of a slice: row R = t >> 1 inside the tile, k-half h = t & 1 (32 weights =
    // two 16-weight units, lane groups g = 2h and 2h + 1)
    int64_t wrow[C::WITEMS];
    int wdst[C::WITEMS];
    Plane<SRC> wpl[C::WITEMS][2];
    uint32_t bword[C::WITEMS], rbase[C::WITEMS];  // raw groups: current bitmap word, raw index at its start
    const uint8_t* pmeta[C::WITEMS];               // direct plane: the item tile's meta row
    u32x2 mcur[C::WITEMS], mnext[C::WITEMS];       // direct plane: meta of this step and the next
#pragma unroll
    for (int it = 0; it < C::WITEMS; it++) {
        const int t = tid + 256 * it, R = t >> 1, h = t & 1;
        const int64_t rr = n0 + R;
        wrow[it] = DIRECT ? rr : (rr < a.N ? rr : a.N - 1);
        wdst[it] = ((R >> 4) * 2 + h) * 64 + (R & 15);  // piece q adds 16 * q
        wpl[it][0] = Plane<SRC>(a, wrow[it], 2 * h);
        wpl[it][1] = Plane<SRC>(a, wrow[it], 2 * h + 1);
        bword[it] = 0;
        rbase[it] = RAW ? a.row_base[wrow[it]] : 0;
        if (DIRECT) {
            int64_t tt = rr >> 4;
            tt = tt < static_cast<int64_t>(a.tiles) ? tt : a.tiles - 1;
            pmeta[it] = a.dmeta + 8 * tt * G;
            mnext[it] = *reinterpret_cast<const u32x2*>(pmeta[it] + 8 * static_cast<int64_t>(j0));
        }
    }
    const uint16_t* xsrc[C::XITEMS];
    bool xok[C::XITEMS];
    int xdst[C::XITEMS];
#pragma unroll
    for (int it = 0; it < C::XITEMS; it++) {
        const int t = tid + 256 * it, R = t >> 1, h = t & 1;
        const int64_t m = m0 + R;
        xok[it] = m < a.M && t < BM * 2;
        xsrc[it] = a.x + (xok[it] ? m : 0) * a.ldx + 32 * h;
        xdst[it] = ((R >> 4) * 2 + h) * 64 + (R & 15);
    }

    floatx4 acc[C::TN][C::TM];
#pragma unroll
    for (int i = 0; i < C::TN; i++)
#pragma unroll
        for (int c = 0; c < C::TM; c++) acc[i][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    W16 wr[C::WITEMS][2];
    u32x4 rsm[C::WITEMS][2], rex[C::WITEMS][2];  // true sign/mantissa + exponents of a raw item
    bool israw[C::WITEMS];
    u32x4 xr[C::XITEMS][4];
    // Issue every global load step j needs. The raw-group decision for step j uses the
    // bitmap word fetched at the last multiple of 32, so a raw item's true data is
    // requested here too, together with the rest, and never from the rebuild.
    auto load_step = [&](uint32_t j) {
#pragma unroll
        for (int it = 0; it < C::WITEMS; it++) {
            if (RAW && (j == j0 || (j & 31) == 0)) {  // once every 32 steps, before this step's other loads
                rbase[it] = j == j0 ? raw_base_at(a, wrow[it], j0) : rbase[it] + __popc(bword[it]);
                bword[it] = a.bitmap[wrow[it] * a.words + (j >> 5)];
            }
        }
#pragma unroll
        for (int it = 0; it < C::WITEMS; it++) {
            wpl[it][0].load(j, wr[it][0]);
            wpl[it][1].load(j, wr[it][1]);
            if (DIRECT) {
                // meta of step j arrived with the previous step; this step's raw exponents
                // ride with its other loads, the next step's meta is requested now
                const int R = (tid + 256 * it) >> 1, h = (tid + 256 * it) & 1;
                mcur[it] = mnext[it];
                israw[it] = (mcur[it].x >> (R & 15)) & 1u;
#pragma unroll
                for (int q = 0; q < 2; q++)
                    rex[it][q] = *raw_exp_addr(a, mcur[it], R & 15, 2 * h + q, a.dmeta);
                if (j + 1 < G) mnext[it] = *reinterpret_cast<const u32x2*>(pmeta[it] + 8 * static_cast<int64_t>(j + 1));
            }
            if (RAW) {
                israw[it] = (bword[it] >> (j & 31)) & 1u;
                if (israw[it]) {
                    const int h = (tid + 256 * it) & 1;
                    uint32_t ri = rbase[it] + __popc(bword[it] & ((1u << (j & 31)) - 1u));
                    ri = ri < a.raw_max ? ri : a.raw_max;
                    const u32x4* sp = reinterpret_cast<const u32x4*>(a.sm + wrow[it] * a.K + 64 * static_cast<int64_t>(j) + 32 * h);
                    const u32x4* ep = reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64 + 32 * h);
                    rsm[it][0] = sp[0];
                    rsm[it][1] = sp[1];
                    rex[it][0] = ep[0];
                    rex[it][1] = ep[1];
                }
            }
        }
#pragma unroll
        for (int it = 0; it < C::XITEMS; it++) {
            if (xok[it]) {
                const u32x4* p = reinterpret_cast<const u32x4*>(xsrc[it] + 64 * static_cast<int64_t>(j));
                xr[it][0] = p[0];
                xr[it][1] = p[1];
                xr[it][2] = p[2];
                xr[it][3] = p[3];
            } else {
#pragma unroll
                for (int q = 0; q < 4; q++) xr[it][q] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_step = [&](int st) {
#pragma unroll
        for (int it = 0; it < C::WITEMS; it++) {
            u32x4* dst = As + st * A_VEC + wdst[it];
#pragma unroll
            for (int q = 0; q < 2; q++) {
                u32x4 p0, p1;
                rebuild16<SRC, CONTIG>(a, wr[it][q], p0, p1);
                if (DIRECT && israw[it]) rebuild16_raw(wr[it][q], rex[it][q], p0, p1);
                if (RAW && israw[it]) {
                    uint32_t ea, eb;
                    split_exps(rex[it][q].x, rex[it][q].y, ea, eb);
                    p0 = piece_from_split(ea, eb, rsm[it][q].x, rsm[it][q].y);
                    split_exps(rex[it][q].z, rex[it][q].w, ea, eb);
                    p1 = piece_from_split(ea, eb, rsm[it][q].z, rsm[it][q].w);
                }
                dst[16 * (2 * q)] = p0;
                dst[16 * (2 * q + 1)] = p1;
            }
        }
#pragma unroll
        for (int it = 0; it < C::XITEMS; it++)
            if (tid + 256 * it < BM * 2)
#pragma unroll
                for (int q = 0; q < 4; q++) Bs[st * B_VEC + xdst[it] + 16 * q] = xr[it][q];
    };

    load_step(j0);
    store_step(0);
    __syncthreads();
    for (uint32_t j = j0; j < j1; j++) {
        const int st = (j - j0) & 1;
        if (j + 1 < j1) load_step(j + 1);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            u32x4 af[C::TN], bf[C::TM];
#pragma unroll
            for (int i = 0; i < C::TN; i++) af[i] = As[st * A_VEC + ((wn * C::TN + i) * 2 + h) * 64 + lane];
#pragma unroll
            for (int c = 0; c < C::TM; c++) bf[c] = Bs[st * B_VEC + ((wm * C::TM + c) * 2 + h) * 64 + lane];
#pragma unroll
            for (int i = 0; i < C::TN; i++)
#pragma unroll
                for (int c = 0; c < C::TM; c++) acc[i][c] = mfma16(af[i], bf[c], acc[i][c]);
        }
        if (j + 1 < j1) store_step(st ^ 1);
        __syncthreads();
    }

    static_assert(BM / 2 * BN * 4 <= C::LDS, "split-K epilogue half tile must fit the LDS");
    if (gridDim.y > 1) {  // one of several K slices
        add_tile<BN, BM, C::TN, C::TM, 256>(a, reinterpret_cast<float*>(lds), acc, n0, m0, wn, wm, lane, tid);
        return;
    }
    if (a.hout) {
        swiglu_tile<BN, BM, C::TN, C::TM, 256>(a, reinterpret_cast<float*>(lds), acc, n0, m0, wn, wm, lane, tid);
        return;
    }
    // lane holds D[4*(lane/16) + q][lane%16] = Y^T: 4 consecutive n of one Y row
#pragma unroll
    for (int i = 0; i < C::TN; i++)
#pragma unroll
        for (int c = 0; c < C::TM; c++)
            store_out(a, m0 + (wm * C::TM + c) * 16 + (lane & 15), n0 + (wn * C::TN + i) * 16 + 4 * (lane >> 4),
                      acc[i][c]);
}

// ------------------------------------------------------------------------- variants
// ------------------------------------------------------------------------- wide
// Large-M kernel. Block = 8 waves computing a 256 (W rows) x 256 (X rows) tile; wave
// (wn, wm) owns 64 x 128 of it = 4 x 8 MFMA tiles of 16x16 (128 accumulators per lane),
// so two waves share each SIMD and one wave's MFMAs overlap the other's loads and
// rebuild. Per 64-k step each thread loads 2 W items (16 weights of one row, as
// compressed bytes) and 2 X items (16 k of one X row), rebuilds the W items to bf16 and
// stores both into an LDS stage laid out in MFMA operand order, [16-row tile][k half]
// [lane] of 16 B, so every fragment read is one conflict-free ds_read_b128. Two stages:
// step j+1 is rebuilt and stored while step j's MFMAs run; its loads are issued as soon
// as step j's registers are free (before the barrier that publishes step j), so they have
// the barrier wait and a whole MFMA phase to arrive. Per MFMA a wave reads 3/8 of the
// LDS bytes a 64 x 64 wave tile needs.
template <int SRC, bool CONTIG>
__global__ void __launch_bounds__(512) gemm_wide(GemmArgs a)
{
    constexpr int BN = 256, BM = 256, ITEMS = 2, NWV = 8;
    constexpr int TN = 4, TM = 8;  // 16x16 tiles per wave
    constexpr bool RAW = SRC == UW_W_IDX;
    constexpr bool DIRECT = SRC == UW_W_DIRECT;
    constexpr int A_VEC = BN * 64 * 2 / 16, STAGE_VEC = A_VEC + BM * 64 * 2 / 16;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    u32x4* const S = reinterpret_cast<u32x4*>(lds);

    const uint32_t tiles_n = static_cast<uint32_t>((a.N + BN - 1) / BN);
    const uint32_t tiles_m = static_cast<uint32_t>((a.M + BM - 1) / BM);
    uint32_t tn, tm;
    tile_of_block(blockIdx.x, gridDim.x, tiles_n, tiles_m, tn, tm);
    const int64_t n0 = static_cast<int64_t>(tn) * BN, m0 = static_cast<int64_t>(tm) * BM;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave >> 1, wm = wave & 1;
    const uint32_t G = static_cast<uint32_t>(a.K >> 6);
    uint32_t j0, j1;
    k_slice(a, G, j0, j1);

    // W item it: row 16 * (wave + 8 it) + r of the tile, weights 16g .. 16g+15 of a group;
    // X item it: X row 16 * (wave + 8 it) + r, k 16g .. 16g+15 of a group
    Plane<SRC> wpl[ITEMS];
    int64_t wrow[ITEMS];
    const uint8_t* pmeta[ITEMS];
    uint32_t bword[ITEMS], rbase[ITEMS];
    u32x2 mnext[ITEMS];
    const uint16_t* xsrc[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; it++) {
        const int i = wave + NWV * it;
        const int64_t rr = n0 + 16 * i + r;
        wrow[it] = DIRECT ? rr : (rr < a.N ? rr : a.N - 1);
        wpl[it] = Plane<SRC>(a, wrow[it], g);
        bword[it] = 0;
        rbase[it] = RAW ? a.row_base[wrow[it]] : 0u;
        if (DIRECT) {
            int64_t t = (n0 >> 4) + i;
            t = t < static_cast<int64_t>(a.tiles) ? t : a.tiles - 1;
            pmeta[it] = a.dmeta + 8 * t * G;
            mnext[it] = *reinterpret_cast<const u32x2*>(pmeta[it] + 8 * static_cast<int64_t>(j0));
        }
        const int64_t m = m0 + 16 * i + r;
        xsrc[it] = a.x + (m < a.M ? m : a.M - 1) * a.ldx + 16 * g;
    }
    // X (and bf16 W) slices are read as whole 128-byte row segments: load q of this wave
    // covers tile rows 8 (4 wave + q) .. +7, lane l takes row + l % 8 and 16 bytes l / 8, so
    // eight consecutive lanes store eight rows of one column of the operand-order LDS
    // stage (distinct banks). A row-sliced operand load would touch twice the cache lines.
    // Load q of this wave covers tile rows 8 (4 wave + q) .. +7: lane l takes row + l / 8 and
    // 16-byte chunk l % 8, so consecutive lanes read consecutive bytes of a row (a wave reads
    // eight whole 128-byte row segments). Chunk kap = 2 g + h goes to fragment block (16-row
    // tile, h) at slot 16 g + (row % 16 ^ 2 g ^ 8 h) instead of 16 g + row % 16: each group of
    // 16 lanes then stores into 16 distinct 16-byte bank groups, and a fragment read (lane
    // 16 g + r of block h reads that slot) still does.
    const uint8_t* xseg[4];
    const uint8_t* wseg[4];
    int sdst[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int rho = 8 * (4 * wave + q) + (lane >> 3), kap = lane & 7;
        const int64_t m = m0 + rho, n = n0 + rho;
        xseg[q] = reinterpret_cast<const uint8_t*>(a.x + (m < a.M ? m : a.M - 1) * a.ldx) + 16 * kap;
        wseg[q] = static_cast<const uint8_t*>(a.wplane) + 2 * (n < a.N ? n : a.N - 1) * a.K + 16 * kap;
        const int gq = kap >> 1, hq = kap & 1;
        sdst[q] = (2 * (rho >> 4) + hq) * 64 + 16 * gq + ((rho & 15) ^ (2 * gq) ^ (8 * hq));
    }
    constexpr bool WSEG = SRC == UW_W_BF16;
    // fragment slot of this lane in a block staged from row segments (X, and bf16 W), per h
    const int fslot[2] = {16 * g + (r ^ (2 * g)), 16 * g + (r ^ (2 * g) ^ 8)};

    floatx4 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
        for (int c = 0; c < TM; c++) acc[i][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    W16 wr[ITEMS];
    u32x4 xr[4], ws[WSEG ? 4 : 1];
    u32x4 rsm[ITEMS], rex[ITEMS];  // raw item: true sign/mantissa (index plane), verbatim exponents
    bool israw[ITEMS];
    auto load_step = [&](uint32_t j) {
#pragma unroll
        for (int it = 0; it < ITEMS; it++) {
            if (RAW && (j == j0 || (j & 31) == 0)) {  // bitmap word of this step, refreshed every 32 steps
                rbase[it] = j == j0 ? raw_base_at(a, wrow[it], j0) : rbase[it] + __popc(bword[it]);
                bword[it] = a.bitmap[wrow[it] * a.words + (j >> 5)];
            }
        }
#pragma unroll
        for (int it = 0; it < ITEMS; it++) {
            if (!WSEG) wpl[it].load(j, wr[it]);
            if (DIRECT) {
                const u32x2 mcur = mnext[it];
                israw[it] = (mcur.x >> r) & 1u;
                rex[it] = *raw_exp_addr(a, mcur, r, g, a.dmeta);
                if (j + 1 < G) mnext[it] = *reinterpret_cast<const u32x2*>(pmeta[it] + 8 * static_cast<int64_t>(j + 1));
            }
            if (RAW) {
                israw[it] = (bword[it] >> (j & 31)) & 1u;
                if (israw[it]) {
                    uint32_t ri = rbase[it] + __popc(bword[it] & ((1u << (j & 31)) - 1u));
                    ri = ri < a.raw_max ? ri : a.raw_max;
                    rsm[it] = *reinterpret_cast<const u32x4*>(a.sm + wrow[it] * a.K + 64 * static_cast<int64_t>(j) + 16 * g);
                    rex[it] = *reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64 + 16 * g);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            xr[q] = *reinterpret_cast<const u32x4*>(xseg[q] + 128 * static_cast<int64_t>(j));
            if (WSEG) ws[WSEG ? q : 0] = *reinterpret_cast<const u32x4*>(wseg[q] + 128 * static_cast<int64_t>(j));
        }
    };
    auto store_step = [&](int st) {
        u32x4* const A = S + st * STAGE_VEC;
        u32x4* const B = A + A_VEC;
#pragma unroll
        for (int it = 0; it < ITEMS; it++) {
            if (WSEG) break;
            const int i = wave + NWV * it;
            u32x4 p0, p1;
            rebuild16<SRC, CONTIG>(a, wr[it], p0, p1);
            if (DIRECT && israw[it]) rebuild16_raw(wr[it], rex[it], p0, p1);
            if (RAW && israw[it]) {
                uint32_t ea, eb;
                split_exps(rex[it].x, rex[it].y, ea, eb);
                p0 = piece_from_split(ea, eb, rsm[it].x, rsm[it].y);
                split_exps(rex[it].z, rex[it].w, ea, eb);
                p1 = piece_from_split(ea, eb, rsm[it].z, rsm[it].w);
            }
            A[(2 * i) * 64 + lane] = p0;
            A[(2 * i + 1) * 64 + lane] = p1;
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            B[sdst[q]] = xr[q];
            if (WSEG) A[sdst[q]] = ws[WSEG ? q : 0];
        }
    };
    auto mma_step = [&](int st) {
        const u32x4* const A = S + st * STAGE_VEC;
        const u32x4* const B = A + A_VEC;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            u32x4 bf[TM];
#pragma unroll
            for (int c = 0; c < TM; c++) bf[c] = B[((TM * wm + c) * 2 + h) * 64 + fslot[h]];
#pragma unroll
            for (int i = 0; i < TN; i++) {
                const u32x4 af = A[((TN * wn + i) * 2 + h) * 64 + (WSEG ? fslot[h] : lane)];
#pragma unroll
                for (int c = 0; c < TM; c++) acc[i][c] = mfma16(af, bf[c], acc[i][c]);
            }
        }
    };

    load_step(j0);
    store_step(0);
    if (j0 + 1 < j1) load_step(j0 + 1);
    __syncthreads();
    for (uint32_t j = j0; j + 1 < j1; j++) {
        const int st = (j - j0) & 1;
        // keep the MFMAs after the loads: sunk into the MFMA sequence (to reuse the
        // fragment registers) the loads would leave too little time to arrive
        __builtin_amdgcn_sched_barrier(0);
        mma_step(st);
        store_step(st ^ 1);
        if (j + 2 < j1) load_step(j + 2);
        __syncthreads();
    }
    mma_step((j1 - 1 - j0) & 1);

    static_assert(BM / 2 * BN * 4 <= 2 * STAGE_VEC * 16, "split-K epilogue half tile must fit the LDS");
    if (gridDim.y > 1) {  // one of several K slices
        add_tile<BN, BM, TN, TM, 512>(a, reinterpret_cast<float*>(lds), acc, n0, m0, wn, wm, lane,
                                      static_cast<int>(threadIdx.x));
        return;
    }
    if (a.hout) {
        swiglu_tile<BN, BM, TN, TM, 512>(a, reinterpret_cast<float*>(lds), acc, n0, m0, wn, wm, lane,
                                         static_cast<int>(threadIdx.x));
        return;
    }
    // lane holds D[4*(lane/16) + q][lane%16] = Y^T: 4 consecutive n of one Y row
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
        for (int c = 0; c < TM; c++)
            store_out(a, m0 + (TM * wm + c) * 16 + (lane & 15), n0 + (TN * wn + i) * 16 + 4 * (lane >> 4), acc[i][c]);
}

// ------------------------------------------------------------------------- dma
// Plain bf16 GEMM for large M (the GEMM half of the full-decode and expand pipelines):
// 256 x 256 output tile of 8 waves (4 x 2, 64 x 128 each), both operands sent from global
// memory straight into LDS with global_load_lds_dwordx4, so no VGPR holds them on the way
// and no LDS store instruction is issued. K advances 64 per step through two 64 KB stages.
//
// LDS layout of one operand in one stage: row rho (0..255) of the tile at 128 rho, its
// 16-byte chunk c (k 8c .. 8c+7 of the step) at slot c ^ ((rho >> 1) & 7): the two rows
// that share a 256-byte bank period, and the rows of other periods, get different slots.
// A transfer covers 1 KB: lane l lands at 16 l, i.e. row 8 i + l / 8, slot l mod 8, so it
// fetches chunk (l mod 8) ^ ((rho >> 1) & 7) of that row; the eight lanes of a row still
// read its whole 128-byte segment. A fragment read (lane 16 g + r: row 16 t + r, chunk
// 4 h + g) hits 16 distinct 16-byte bank groups in every 16 lanes.
//
// One barrier per step, placed where every fragment of the step is already in registers:
// after it, the stage the step used takes the transfers of the step after next, the X
// fragments of the next step's first k-half are read, and the step's second k-half is
// multiplied from registers meanwhile, so the matrix cores do not wait for LDS reads at
// the start of a step.
template <int BM, int NST>
__global__ void __launch_bounds__(512) gemm_dma(GemmArgs a)
{
    constexpr int BN = 256, NWV = 8;
    constexpr int TN = 4, TM = BM / 32;  // 16-row W and X tiles per wave (waves 4 along N, 2 along M)
    constexpr int OPB = BN * 128;        // W of one stage
    constexpr int OPX = BM * 128;        // X of one stage
    constexpr int STAGE = OPB + OPX;
    constexpr int NLD = BN / 8 / NWV;    // W transfers per wave per step
    constexpr int NLX = BM / 8 / NWV;    // X transfers per wave per step
    static_assert(NST >= 2 && NST * STAGE <= 160 * 1024 && NLX >= 1, "stage shape");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const uint32_t tiles_n = static_cast<uint32_t>((a.N + BN - 1) / BN);
    const uint32_t tiles_m = static_cast<uint32_t>((a.M + BM - 1) / BM);
    uint32_t tn, tm;
    tile_of_block(blockIdx.x, gridDim.x, tiles_n, tiles_m, tn, tm);
    const int64_t n0 = static_cast<int64_t>(tn) * BN, m0 = static_cast<int64_t>(tm) * BM;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave >> 1, wm = wave & 1;
    const uint32_t G = static_cast<uint32_t>(a.K >> 6);
    uint32_t j0, j1;
    k_slice(a, G, j0, j1);

    // per-lane byte offsets of this wave's transfers (rows past N or M read the last row;
    // the host keeps every offset below 2^32)
    uint32_t woff[NLD], xoff[NLX];
#pragma unroll
    for (int q = 0; q < NLD; q++) {
        const int rho = 8 * (NLD * wave + q) + (lane >> 3);
        const int kap = (lane & 7) ^ ((rho >> 1) & 7);
        const int64_t n = n0 + rho < a.N ? n0 + rho : a.N - 1;
        woff[q] = static_cast<uint32_t>(2 * n * a.K + 16 * kap);
    }
#pragma unroll
    for (int q = 0; q < NLX; q++) {
        const int rho = 8 * (NLX * wave + q) + (lane >> 3);
        const int kap = (lane & 7) ^ ((rho >> 1) & 7);
        const int64_t m = m0 + rho < a.M ? m0 + rho : a.M - 1;
        xoff[q] = static_cast<uint32_t>(2 * m * a.ldx + 16 * kap);
    }
    const uint32_t lds0 = lds_offset(lds);
    const uint8_t* const wbase = static_cast<const uint8_t*>(a.wplane);
    const uint8_t* const xbase = reinterpret_cast<const uint8_t*>(a.x);
    auto issue = [&](uint32_t j, int st) {
        const uint8_t* wb = wbase + 128 * static_cast<int64_t>(j);
        const uint8_t* xb = xbase + 128 * static_cast<int64_t>(j);
        const uint32_t dst = lds0 + st * STAGE;
#pragma unroll
        for (int q = 0; q < NLD; q++) dma16(wb, woff[q], dst + 1024 * (NLD * wave + q));
#pragma unroll
        for (int q = 0; q < NLX; q++) dma16(xb, xoff[q], dst + OPB + 1024 * (NLX * wave + q));
    };
    // fragment slots of this lane for the two k-halves
    const int foff0 = 128 * r + 16 * ((0 + g) ^ ((r >> 1) & 7));
    const int foff1 = 128 * r + 16 * ((4 + g) ^ ((r >> 1) & 7));
    auto bfrags = [&](const uint8_t* S, int fo, u32x4 (&bf)[TM]) {
#pragma unroll
        for (int c = 0; c < TM; c++)
            bf[c] = *reinterpret_cast<const u32x4*>(S + OPB + 2048 * (TM * wm + c) + fo);
    };
    auto afrag = [&](const uint8_t* S, int fo, int i) {
        return *reinterpret_cast<const u32x4*>(S + 2048 * (TN * wn + i) + fo);
    };

    floatx4 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
        for (int c = 0; c < TM; c++) acc[i][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    u32x4 bf0[TM], an;
    if (j0 < j1) {
        issue(j0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int p = 1; p < NST; p++)
            if (j0 + p < j1) issue(j0 + p, p);
        bfrags(lds, foff0, bf0);
        an = afrag(lds, foff0, 0);
    }
    for (uint32_t j = j0; j < j1; j++) {
        const int st = (j - j0) % NST, sn = (st + 1) % NST;
        const uint8_t* S = lds + st * STAGE;
        // first k-half from the X fragments already in registers; the rest of the step's
        // fragments are read meanwhile (W one tile ahead of its MFMAs)
        u32x4 a1[TN], bf1[TM];
#pragma unroll
        for (int i = 0; i < TN; i++) {
            const u32x4 ac = an;
            if (i + 1 < TN) an = afrag(S, foff0, i + 1);
            a1[i] = afrag(S, foff1, i);
            if (i == 0) bfrags(S, foff1, bf1);
#pragma unroll
            for (int c = 0; c < TM; c++) acc[i][c] = mfma16(ac, bf0[c], acc[i][c]);
        }
        // every wave holds all of this step's fragments and (after the wait) its transfers
        // of the next step have landed: after the barrier this stage takes the step after
        // next, and the next step's first X fragments are read. (Unconditional, also in
        // the last step: behind a branch the compiler would make the second k-half's
        // MFMAs wait for those reads. The scheduling barriers keep the second k-half's
        // MFMAs after the barrier and the reads, where they hide the reads' latency.)
        __builtin_amdgcn_sched_barrier(0);
        // (with NST stages the NST - 2 steps after the next may still be in flight)
        if (NST > 2 && j + NST - 1 < j1) {
            constexpr int younger = (NST > 2 ? NST - 2 : 0) * (NLD + NLX);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(younger) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        if (j + NST < j1) issue(j + NST, st);
        bfrags(lds + sn * STAGE, foff0, bf0);
        an = afrag(lds + sn * STAGE, foff0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TN; i++)
#pragma unroll
            for (int c = 0; c < TM; c++) acc[i][c] = mfma16(a1[i], bf1[c], acc[i][c]);
    }

    static_assert(BM / 2 * BN * 4 <= NST * STAGE, "split-K epilogue half tile must fit the LDS");
    if (gridDim.y > 1) {  // one of several K slices
        add_tile<BN, BM, TN, TM, 64 * NWV>(a, reinterpret_cast<float*>(lds), acc, n0, m0, wn, wm, lane,
                                           static_cast<int>(threadIdx.x));
        return;
    }
    if (a.hout) {
        swiglu_tile<BN, BM, TN, TM, 64 * NWV>(a, reinterpret_cast<float*>(lds), acc, n0, m0, wn, wm, lane,
                                              static_cast<int>(threadIdx.x));
        return;
    }
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
        for (int c = 0; c < TM; c++)
            store_out(a, m0 + (TM * wm + c) * 16 + (lane & 15), n0 + (TN * wn + i) * 16 + 4 * (lane >> 4), acc[i][c]);
}

struct Variant {
    const char* name;
    int kind;  // 0 skinny, 1 tiled, 2 wide, 3 dma (bf16 W, both operands by LDS DMA)
    int rt, nw, u;
    int bn, bm;
    int xnear;  // skinny: X one group ahead in one register set instead of with the ring
    int xt;     // skinny: X read as whole row segments and put in operand order through LDS:
                // 1 staged in registers ("xt"), 2 by LDS DMA into a ring of tiles ("xd")
    int ks;     // skinny: K cut into slices so that row blocks x slices fill the CUs (fp32 atomics into Y)
};

const Variant kVariants[] = {
    {"skinny rt1 u8 w4", 0, 1, 4, 8, 0, 0},  {"skinny rt1 u4 w8", 0, 1, 8, 4, 0, 0},
    {"skinny rt1 u4 w4", 0, 1, 4, 4, 0, 0},  {"skinny rt2 u4 w4", 0, 2, 4, 4, 0, 0},
    {"skinny rt2 u4 w8", 0, 2, 8, 4, 0, 0},  {"skinny rt4 u2 w4", 0, 4, 4, 2, 0, 0},
    {"tiled 128x128", 1, 0, 0, 0, 128, 128}, {"tiled 128x64", 1, 0, 0, 0, 128, 64},
    {"tiled 256x128", 1, 0, 0, 0, 256, 128}, {"wide 256x256", 2, 0, 0, 0, 256, 256},
    {"skinny rt4 u4 w4", 0, 4, 4, 4, 0, 0},  {"skinny rt4 u2 w8 x1", 0, 4, 8, 2, 0, 0, 1},
    {"skinny rt4 u2 w4 x1", 0, 4, 4, 2, 0, 0, 1}, {"skinny rt2 u4 w8 x1", 0, 2, 8, 4, 0, 0, 1},
    {"skinny rt4 u2 w4 xt", 0, 4, 4, 2, 0, 0, 0, 1}, {"skinny rt4 u4 w4 xt", 0, 4, 4, 4, 0, 0, 0, 1},
    {"skinny rt2 u4 w4 xt", 0, 2, 4, 4, 0, 0, 0, 1},
    {"skinny rt4 u2 w4 ks", 0, 4, 4, 2, 0, 0, 0, 0, 1}, {"skinny rt4 u2 w4 xt ks", 0, 4, 4, 2, 0, 0, 0, 1, 1},
    {"skinny rt4 u2 w8 xd", 0, 4, 8, 2, 0, 0, 0, 2},    {"skinny rt4 u2 w4 xd", 0, 4, 4, 2, 0, 0, 0, 2},
    {"skinny rt4 u2 w8 xd ks", 0, 4, 8, 2, 0, 0, 0, 2, 1},
    {"dma 256x256", 3, 0, 8, 2, 256, 256},              {"dma 256x128 s3", 3, 0, 8, 3, 256, 128},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

// Raise a kernel's dynamic LDS limit past the 64 KB default (gfx950 has 160 KB per CU),
// once per device (bit d of `done`; a lost update between racing threads only repeats the
// call).
hipError_t allow_lds(const void* fn, size_t bytes, uint64_t& done)
{
    if (bytes <= 64 * 1024) return hipSuccess;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if ((done >> dev) & 1u) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
    if (e == hipSuccess) done |= uint64_t{1} << dev;
    return e;
}

template <int SRC, bool CONTIG, int CT, int RT, int U, int NW, bool XNEAR, int XT>
hipError_t launch_skinny_ct(const GemmArgs& g, hipStream_t s)
{
    const uint32_t G = static_cast<uint32_t>(g.K / 64);
    const uint32_t ks = g.kgroups ? (G + g.kgroups - 1) / g.kgroups : 1;
    const dim3 grid(static_cast<uint32_t>((g.N + 16 * RT - 1) / (16 * RT)), ks);
    constexpr size_t lds = skinny_lds<CT, RT, U, NW, XT>();
    static uint64_t attr_done = 0;  // devices the LDS limit was raised on
    hipError_t e = allow_lds(reinterpret_cast<const void*>(&gemm_skinny<SRC, CONTIG, CT, RT, U, NW, XNEAR, XT>), lds, attr_done);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_skinny<SRC, CONTIG, CT, RT, U, NW, XNEAR, XT>), grid, dim3(64 * NW), lds, s, g);
    return hipGetLastError();
}

template <int SRC, bool CONTIG, int RT, int U, int NW, bool XNEAR = false, int XT = 0>
hipError_t launch_skinny_rt(const GemmArgs& g, hipStream_t s)
{
    const int ct = static_cast<int>((g.M + 15) / 16);
    switch (ct) {
    case 1: return launch_skinny_ct<SRC, CONTIG, 1, RT, U, NW, XNEAR, XT>(g, s);
    case 2: return launch_skinny_ct<SRC, CONTIG, 2, RT, U, NW, XNEAR, XT>(g, s);
    default: return launch_skinny_ct<SRC, CONTIG, 4, RT, U, NW, XNEAR, XT>(g, s);
    }
}

// Work split of the tiled and wide kernels over K. With few output tiles (down_proj-like
// shapes: small N, long K) the CUs would idle, so K is cut into ks slices of whole
// 64-groups, one workgroup each; Y is zeroed first and every slice adds its partial tile
// into Y with fp32 atomics. ks is the minimum of a small time model fitted to this
// kernel's own measurements on the 256-CU part: a workgroup of S steps takes
// c0 + c1 * S microseconds, `cap` workgroups run at once, and each sliced output element
// costs `atom` microseconds per slice in L2 atomics.
struct SliceModel {
    uint32_t per_cu;  // resident workgroups per CU (LDS / register bound)
    double c0, c1;    // us per workgroup, us per 64-group step
};
constexpr SliceModel kTiledModel = {2, 3.2, 1.66};  // 128 x 128 tile, 4 waves
constexpr SliceModel kWideModel = {1, 22.0, 2.07};   // 256 x 256 tile, 8 waves
constexpr SliceModel kDmaModel = {1, 22.0, 1.75};    // 256 x 256 tile, operands by LDS DMA
constexpr double kAtomUs = 3.3e-6;

struct SlicePlan {
    uint32_t ks;
    double us;
};

SlicePlan plan_slices(const SliceModel& mdl, int64_t N, int64_t K, int64_t M, int64_t bn, int64_t bm)
{
    const uint32_t G = static_cast<uint32_t>(K / 64);
    const uint64_t tiles = static_cast<uint64_t>(((N + bn - 1) / bn) * ((M + bm - 1) / bm));
    const uint64_t cap = static_cast<uint64_t>(mdl.per_cu) * cu_count();
    uint32_t most = G / 8;
    most = most < 1 ? 1 : most > 64 ? 64 : most;
    SlicePlan best = {1, 1e300};
    for (uint32_t ks = 1; ks <= most; ks++) {
        const uint32_t kg = (G + ks - 1) / ks;
        if (ks > 1 && (G + kg - 1) / kg != ks) continue;  // same groups per slice as a smaller ks
        const uint64_t waves = (tiles * ks + cap - 1) / cap;
        const double us = waves * (mdl.c0 + mdl.c1 * kg) + (ks > 1 ? kAtomUs * ks * M * N : 0.0);
        if (us < best.us) best = {ks, us};
    }
    return best;
}

// K slices of a launch whose arguments carry kgroups (0 = one slice).
uint32_t slices_of(const GemmArgs& g)
{
    const uint32_t G = static_cast<uint32_t>(g.K / 64);
    return g.kgroups ? (G + g.kgroups - 1) / g.kgroups : 1;
}

hipError_t launch_sliced(const void* fn, GemmArgs g, uint32_t tiles, uint32_t threads, size_t lds, hipStream_t s)
{
    void* args[] = {&g};
    return hipLaunchKernel(fn, dim3(tiles, slices_of(g)), dim3(threads), args, lds, s);
}

template <int SRC, bool CONTIG, int BN, int BM>
hipError_t launch_tiled_t(const GemmArgs& g, hipStream_t s)
{
    using C = TiledCfg<BN, BM>;
    static uint64_t attr_done = 0;  // devices the LDS limit was raised on
    const void* fn = reinterpret_cast<const void*>(&gemm_tiled<SRC, CONTIG, BN, BM>);
    hipError_t e = allow_lds(fn, C::LDS, attr_done);
    if (e != hipSuccess) return e;
    const uint32_t tiles = static_cast<uint32_t>(((g.N + BN - 1) / BN) * ((g.M + BM - 1) / BM));
    e = launch_sliced(fn, g, tiles, 256, C::LDS, s);
    return e != hipSuccess ? e : hipGetLastError();
}

template <int BM, int NST>
hipError_t launch_dma(const GemmArgs& g, hipStream_t s)
{
    constexpr size_t lds = NST * (256 + BM) * 128;
    static uint64_t attr_done = 0;  // devices the LDS limit was raised on
    const void* fn = reinterpret_cast<const void*>(&gemm_dma<BM, NST>);
    hipError_t e = allow_lds(fn, lds, attr_done);
    if (e != hipSuccess) return e;
    const uint32_t tiles = static_cast<uint32_t>(((g.N + 255) / 256) * ((g.M + BM - 1) / BM));
    e = launch_sliced(fn, g, tiles, 512, lds, s);
    return e != hipSuccess ? e : hipGetLastError();
}

// The 256 x 256 DMA GEMM in whole rounds of the CUs. When its tiles leave a last round that
// only part of the CUs would run (the gate shape at M = 4096: 896 tiles = 3.5 rounds of 256),
// the column blocks of that round go to a second launch of the 256 x 128 kernel, whose
// half-height tiles finish a round in a little over half the time. Both launches sum every
// output over K in the same order, so Y is the same as from one launch.
hipError_t launch_dma_rounds(const GemmArgs& g, hipStream_t s)
{
    const int64_t tn = (g.N + 255) / 256, tm = (g.M + 255) / 256, cus = cu_count();
    if (g.kgroups == 0 && tn * tm > cus && (tn * tm) % cus != 0) {
        int64_t nm = tn * tm / cus * cus / tm;  // column blocks of the first launch: whole rounds
        while (nm > 0 && (nm * tm) % cus != 0) nm--;
        const int64_t n0 = nm * 256;
        if (nm > 0 && n0 < g.N && (tn - nm) * ((g.M + 127) / 128) <= cus) {
            GemmArgs a = g;
            a.N = n0;
            hipError_t e = launch_dma<256, 2>(a, s);
            if (e != hipSuccess) return e;
            GemmArgs b = g;
            b.N = g.N - n0;
            b.wplane = static_cast<const uint8_t*>(g.wplane) + 2 * n0 * g.K;
            b.y = g.y + n0;
            b.hout = g.hout ? g.hout + n0 : nullptr;
            return launch_dma<128, 3>(b, s);
        }
    }
    return launch_dma<256, 2>(g, s);
}

template <int SRC, bool CONTIG>
hipError_t launch_wide_t(const GemmArgs& g, hipStream_t s)
{
    constexpr size_t lds = 2 * (256 + 256) * 64 * 2;
    static uint64_t attr_done = 0;  // devices the LDS limit was raised on
    hipError_t e = allow_lds(reinterpret_cast<const void*>(&gemm_wide<SRC, CONTIG>), lds, attr_done);
    if (e != hipSuccess) return e;
    const uint32_t tiles = static_cast<uint32_t>(((g.N + 255) / 256) * ((g.M + 255) / 256));
    e = launch_sliced(reinterpret_cast<const void*>(&gemm_wide<SRC, CONTIG>), g, tiles, 512, lds, s);
    return e != hipSuccess ? e : hipGetLastError();
}

// K slices of a skinny "ks" launch: as many as it takes for row blocks x slices to fill the
// CUs, each slice at least 8 groups (1 = no split).
uint32_t skinny_slices(int64_t N, int64_t K, int rt)
{
    const uint32_t G = static_cast<uint32_t>(K / 64);
    const uint32_t blocks = static_cast<uint32_t>((N + 16 * rt - 1) / (16 * rt));
    uint32_t ks = cu_count() / (blocks ? blocks : 1);
    const uint32_t most = G / 8 ? G / 8 : 1;
    ks = ks < 1 ? 1 : ks > most ? most : ks;
    const uint32_t kg = (G + ks - 1) / ks;
    return (G + kg - 1) / kg;
}

// The K slices a launch of variant v uses on (N, K, M): split_k when it is positive, else
// the variant's own choice (the time model for the 128x128 and 256x256 tiles, enough
// slices to fill the CUs for the skinny "ks" variants, none for the others), rounded so
// that every slice has the same whole number of 64-groups.
uint32_t resolve_split(const Variant& v, int64_t N, int64_t K, int64_t M, int32_t split_k)
{
    const uint32_t G = static_cast<uint32_t>(K / 64);
    uint32_t ks;
    if (split_k > 0)
        ks = static_cast<uint32_t>(split_k);
    else if (v.kind == 0)
        ks = v.ks ? skinny_slices(N, K, v.rt) : 1;
    else if (v.kind == 1)
        ks = v.bn == 128 && v.bm == 128 ? plan_slices(kTiledModel, N, K, M, 128, 128).ks : 1;
    else
        ks = plan_slices(v.kind == 3 ? kDmaModel : kWideModel, N, K, M, 256, v.kind == 3 ? v.bm : 256).ks;
    ks = ks < 1 ? 1 : ks > G ? G : ks;
    const uint32_t kg = (G + ks - 1) / ks;
    return (G + kg - 1) / kg;
}

template <int SRC, bool CONTIG>
hipError_t launch_src(const GemmArgs& g, const Variant& v, hipStream_t s)
{
    if (v.kind == 2) return launch_wide_t<SRC, CONTIG>(g, s);
    if (v.kind == 3) {
        if constexpr (SRC == UW_W_BF16) return v.bm == 128 ? launch_dma<128, 3>(g, s) : launch_dma_rounds(g, s);
        return hipErrorNotSupported;  // (rejected before: bf16 weights only)
    }
    // (a "ks" variant is its neighbour's kernel with a K split chosen for it; the split is
    // in g.kgroups, set by the caller)
    if (v.kind == 0) {
        if (v.rt == 1 && v.u == 8) return launch_skinny_rt<SRC, CONTIG, 1, 8, 4>(g, s);
        if (v.rt == 1 && v.nw == 8) return launch_skinny_rt<SRC, CONTIG, 1, 4, 8>(g, s);
        if (v.rt == 1) return launch_skinny_rt<SRC, CONTIG, 1, 4, 4>(g, s);
        if (v.rt == 2 && v.nw == 8) return launch_skinny_rt<SRC, CONTIG, 2, 4, 8>(g, s);
        if (v.rt == 2) return launch_skinny_rt<SRC, CONTIG, 2, 4, 4>(g, s);
        if (v.xt == 2) {
            if constexpr (SRC == UW_W_DIRECT) {
                if (v.nw == 8) return launch_skinny_rt<SRC, CONTIG, 4, 2, 8, false, 2>(g, s);
                return launch_skinny_rt<SRC, CONTIG, 4, 2, 4, false, 2>(g, s);
            }
            return hipErrorNotSupported;  // (rejected before: direct planes only)
        }
        if (v.xt && v.rt == 4 && v.u == 4) return launch_skinny_rt<SRC, CONTIG, 4, 4, 4, false, 1>(g, s);
        if (v.xt && v.rt == 4) return launch_skinny_rt<SRC, CONTIG, 4, 2, 4, false, 1>(g, s);
        if (v.xt) return launch_skinny_rt<SRC, CONTIG, 2, 4, 4, false, 1>(g, s);
        if (v.xnear && v.rt == 4 && v.nw == 8) return launch_skinny_rt<SRC, CONTIG, 4, 2, 8, true>(g, s);
        if (v.xnear && v.rt == 4) return launch_skinny_rt<SRC, CONTIG, 4, 2, 4, true>(g, s);
        if (v.xnear) return launch_skinny_rt<SRC, CONTIG, 2, 4, 8, true>(g, s);
        if (v.rt == 4 && v.u == 4) return launch_skinny_rt<SRC, CONTIG, 4, 4, 4>(g, s);
        return launch_skinny_rt<SRC, CONTIG, 4, 2, 4>(g, s);
    }
    if (v.bn == 128 && v.bm == 128) return launch_tiled_t<SRC, CONTIG, 128, 128>(g, s);
    if (v.bn == 128 && v.bm == 64) return launch_tiled_t<SRC, CONTIG, 128, 64>(g, s);
    return launch_tiled_t<SRC, CONTIG, 256, 128>(g, s);
}

template <int CT, int RT, int U, int NW, bool XNEAR, int XT, int PAIR>
hipError_t launch_gate_up_p(const GateUpArgs& ga, hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>((ga.gate.N + 16 * RT - 1) / (16 * RT)));
    constexpr size_t lds = skinny_lds<CT, RT, U, NW, XT, PAIR>() + static_cast<size_t>(RT) * CT * 256 * 4;
    if constexpr (lds > 160 * 1024) {
        (void)ga;
        (void)s;
        (void)grid;
        return hipErrorNotSupported;  // (8 waves with X rings beside the reduction at M > 32)
    } else {
        const void* fn = reinterpret_cast<const void*>(&gemm_skinny_gate_up<true, true, CT, RT, U, NW, XNEAR, XT, PAIR>);
        static uint64_t attr_done = 0;  // devices the LDS limit was raised on
        hipError_t e = allow_lds(fn, lds, attr_done);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((gemm_skinny_gate_up<true, true, CT, RT, U, NW, XNEAR, XT, PAIR>), grid, dim3(64 * NW), lds, s, ga);
        return hipGetLastError();
    }
}

// 4 waves take group j of gate and up in one step (X fetched once for both; 2 RT row tiles
// per slot, which fits the 512 registers of a lone wave per SIMD); 8 waves, two per SIMD
// with half the registers each, stream gate's groups and then up's through one ring.
template <int CT, int RT, int U, int NW, bool XNEAR, int XT>
hipError_t launch_gate_up_ct(const GateUpArgs& ga, hipStream_t s)
{
    return launch_gate_up_p<CT, RT, U, NW, XNEAR, XT, NW == 4 ? 2 : 1>(ga, s);
}

template <int RT, int U, int NW, bool XNEAR = false, int XT = 0>
hipError_t launch_gate_up_rt(const GateUpArgs& ga, hipStream_t s)
{
    const int ct = static_cast<int>((ga.gate.M + 15) / 16);
    switch (ct) {
    case 1: return launch_gate_up_ct<1, RT, U, NW, XNEAR, XT>(ga, s);
    case 2: return launch_gate_up_ct<2, RT, U, NW, XNEAR, XT>(ga, s);
    default: return launch_gate_up_ct<4, RT, U, NW, XNEAR, XT>(ga, s);
    }
}

// The skinny variants with a fused gate/up form (the defaults for M <= 64 and their
// neighbours); the others return hipErrorNotSupported.
hipError_t launch_gate_up(const GateUpArgs& ga, const Variant& v, hipStream_t s)
{
    if (v.kind != 0) return hipErrorNotSupported;
    // one K slice only (a "ks" variant that cuts nothing on this shape is its unsplit
    // neighbour, which has a fused form)
    if (ga.gate.kgroups || ga.up.kgroups) return hipErrorNotSupported;
    if (v.xt == 2 && v.nw == 8) return launch_gate_up_rt<4, 2, 8, false, 2>(ga, s);
    if (v.xt == 2) return launch_gate_up_rt<4, 2, 4, false, 2>(ga, s);
    if (v.xt && v.rt == 4 && v.u == 2 && v.nw == 4) return launch_gate_up_rt<4, 2, 4, false, 1>(ga, s);
    if (v.xt || v.xnear) return hipErrorNotSupported;
    if (v.rt == 4 && v.u == 2 && v.nw == 4) return launch_gate_up_rt<4, 2, 4>(ga, s);
    if (v.rt == 2 && v.u == 4 && v.nw == 4) return launch_gate_up_rt<2, 4, 4>(ga, s);
    if (v.rt == 1 && v.u == 4 && v.nw == 4) return launch_gate_up_rt<1, 4, 4>(ga, s);
    if (v.rt == 1 && v.u == 4 && v.nw == 8) return launch_gate_up_rt<1, 4, 8>(ga, s);
    return hipErrorNotSupported;
}

}  // namespace

uw_status make_args(const uw_gemm_args* p, GemmArgs& g, bool& contig, int& v);

uw_status launch_gate_up_gemm(const uw_gemm_args* gate, const uw_gemm_args* up, uint16_t* d_h, int64_t ldh,
                              void* stream, const ZeroTarget* clear)
{
    clear_error();
    if (!gate || !up || !gate->h || !up->h) return fail(UW_EINVAL, "NULL argument");
    if (gate->src != UW_W_DIRECT || up->src != UW_W_DIRECT)
        return fail(UW_EUNSUPPORTED, "the fused gate/up GEMM takes direct planes only");
    if (gate->M != up->M || gate->h->N != up->h->N || gate->h->K != up->h->K)
        return fail(UW_ESHAPE, "gate and up must have the same M, N and K");
    if (gate->d_x != up->d_x || gate->ldx != up->ldx) return fail(UW_EINVAL, "gate and up must read the same X");
    if (gate->M < 0) return fail(UW_ESHAPE, "M < 0");
    if (gate->M == 0) return UW_OK;
    if (gate->M > 64) return fail(UW_EUNSUPPORTED, "the fused gate/up GEMM takes M <= 64");
    if (!d_h || !aligned(d_h, 2)) return fail(UW_EINVAL, "NULL or misaligned d_h");
    if (ldh < gate->h->N) return fail(UW_EINVAL, "ldh must be >= N");
    GateUpArgs ga;
    bool cg = false, cu = false;
    int vg = 0, vu = 0;
    uw_gemm_args upv = *up;
    upv.variant = gate->variant;  // one launch, one variant and split: the gate's
    upv.split_k = gate->split_k;
    uw_status st = make_args(gate, ga.gate, cg, vg);
    if (st == UW_OK) st = make_args(&upv, ga.up, cu, vu);
    if (st != UW_OK) return st;
    if (!cg || !cu) return fail(UW_EUNSUPPORTED, "the fused gate/up GEMM needs palettes of consecutive exponents");
    ga.h = d_h;
    ga.ldh = ldh;
    ga.zy = nullptr;
    ga.zld = 0;
    ga.zM = ga.zN = 0;
    if (clear && clear->y && clear->M > 0 && clear->N > 0) {
        if (!aligned(clear->y, 16) || clear->ld % 4 || clear->ld < clear->N || clear->M * ((clear->N + 3) / 4) >= (int64_t{1} << 32))
            return fail(UW_EINVAL, "bad Y to clear");
        ga.zy = clear->y;
        ga.zld = clear->ld;
        ga.zM = static_cast<uint32_t>(clear->M);
        ga.zN = static_cast<uint32_t>(clear->N);
    }
    const hipError_t e = launch_gate_up(ga, kVariants[vg], static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return fail(UW_EUNSUPPORTED, "variant %d has no fused gate/up form", vg);
    if (e != hipSuccess) return fail(UW_EHIP, "gate/up launch failed: %s", hipGetErrorString(e));
    return UW_OK;
}

int default_variant(int64_t N, int64_t K, int64_t M, int32_t src)
{
    if (M <= 64) {
        // the most rows per workgroup (X reused across more weight rows) that still gives
        // ~200 workgroups of 16 * rt rows
        const int64_t tiles = (N + 15) / 16;  // 16-row tiles
        if (tiles >= 4 * 200) return M > 16 ? 14 : 5;  // rt4 u2 w4 (xt: X through LDS)
        if (tiles >= 2 * 200) return 3;                // rt2 u4 w4
        return M > 16 ? 2 : 1;                // rt1 u4 w4 / rt1 u4 w8
    }
    // the 128 x 128 or the 256 x 256 kernel, each with its best K split (for bf16 weights
    // the 256 x 256 tile fed by LDS DMA, the last variant)
    const double t_tiled = plan_slices(kTiledModel, N, K, M, 128, 128).us;
    if (src == UW_W_BF16 && 2 * N * K < (int64_t{1} << 32) && 2 * M * K < (int64_t{1} << 32)) {
        const double t_dma = plan_slices(kDmaModel, N, K, M, 256, 256).us;
        int dma = 9;  // the 256 x 256 DMA variant
        for (int v = 0; v < kNumVariants; v++)
            if (kVariants[v].kind == 3 && kVariants[v].bm == 256) dma = v;
        return t_dma < t_tiled ? dma : 6;
    }
    const double t_wide = plan_slices(kWideModel, N, K, M, 256, 256).us;
    return t_wide < t_tiled ? 9 : 6;
}

// Validate one GEMM's arguments and fill its kernel arguments; v = the variant to run.
uw_status make_args(const uw_gemm_args* p, GemmArgs& g, bool& contig, int& v)
{
    if (!p || !p->h) return fail(UW_EINVAL, "NULL argument");
    const uw_header* h = p->h;
    if (p->M < 0) return fail(UW_ESHAPE, "M < 0");
    if (h->N < 1 || h->K < 1 || h->K % 64) return fail(UW_ESHAPE, "bad W shape");
    if (!p->d_x || !p->d_y || !p->d_wplane) return fail(UW_EINVAL, "NULL device pointer");
    if (p->ldx < h->K || p->ldx % 8) return fail(UW_EINVAL, "ldx must be >= K and a multiple of 8");
    if (p->ldy < h->N) return fail(UW_EINVAL, "ldy must be >= N");
    if (!aligned(p->d_x, 16) || !aligned(p->d_y, 16) || !aligned(p->d_wplane, 16))
        return fail(UW_EINVAL, "device pointers must be 16-byte aligned");
    if (p->src < UW_W_BF16 || p->src > UW_W_DIRECT) return fail(UW_EINVAL, "bad src %d", p->src);
    v = p->variant < 0 ? default_variant(h->N, h->K, p->M, p->src) : p->variant;
    if (v >= kNumVariants) return fail(UW_EINVAL, "variant %d out of range", v);
    if (!uw_variant_supports(v, h->N, h->K, p->M, p->src)) return fail(UW_EUNSUPPORTED, "variant %d does not support this problem", v);
    if (p->split_k < 0 || p->split_k > h->K / 64) return fail(UW_EINVAL, "split_k %d outside 0..K/64", p->split_k);
    if (kVariants[v].kind == 0 && 2 * p->M * p->ldx + 32 * h->K >= (int64_t{1} << 32))
        return fail(UW_EUNSUPPORTED, "variant %d addresses X and W with 32-bit offsets: ldx or K too large", v);
    if (kVariants[v].kind == 3 && (2 * p->M * p->ldx >= (int64_t{1} << 32) || 2 * h->N * h->K >= (int64_t{1} << 32)))
        return fail(UW_EUNSUPPORTED, "variant %d addresses X and W with 32-bit offsets: X or W too large", v);
    std::memset(&g, 0, sizeof g);
    g.x = p->d_x;
    g.wplane = p->d_wplane;
    g.y = p->d_y;
    g.ldx = p->ldx;
    g.ldy = p->ldy;
    g.M = p->M;
    g.N = h->N;
    g.K = h->K;
    const uint32_t G = static_cast<uint32_t>(h->K / 64);
    const uint32_t ks = resolve_split(kVariants[v], h->N, h->K, p->M, p->split_k);
    g.kgroups = ks > 1 ? (G + ks - 1) / ks : 0;  // zero: one slice, Y written, not added into
    contig = false;
    if (p->src != UW_W_BF16) {
        if (!p->d_blob) return fail(UW_EINVAL, "d_blob needed for this src");
        uw_status st = check_header(h, h->total_bytes);
        if (st != UW_OK) return st;
        if (!aligned(p->d_blob, 256)) return fail(UW_EINVAL, "d_blob must be 256-byte aligned");
        const uint8_t* b = static_cast<const uint8_t*>(p->d_blob);
        g.sm = b + h->off_sm;
        g.bitmap = reinterpret_cast<const uint32_t*>(b + h->off_bitmap);
        g.row_base = reinterpret_cast<const uint32_t*>(b + h->off_rowbase);
        g.raw = b + h->off_raw;
        g.words = h->bitmap_words;
        g.raw_max = h->n_raw > 0 ? static_cast<uint32_t>(h->n_raw - 1) : 0;
        std::memcpy(g.pal, h->palette, 16);
        ValueOrder vo;
        value_order(h, &vo);
        std::memcpy(g.vpal, vo.sorted, 16);
        g.base4 = vo.sorted[0] * 0x01010101u;
        contig = vo.contiguous;
        const uint64_t T = static_cast<uint64_t>((h->N + 15) / 16), G = static_cast<uint64_t>(h->K / 64);
        g.tiles = static_cast<uint32_t>(T);
        g.dmeta = static_cast<const uint8_t*>(p->d_wplane) + 1536 * T * G;
        // with no raw group the side table is empty: point it at the meta section (at least
        // 64 readable bytes) so that a clamped index still reads inside the plane
        g.dside = h->n_raw > 0 ? g.dmeta + (8 * T * G + 63) / 64 * 64 : g.dmeta;
    }
    return UW_OK;
}

uw_status launch_expand_direct(const uw_header* h, const uint8_t* d_direct, uint16_t* d_w, void* stream)
{
    clear_error();
    if (!h || !d_direct || !d_w) return fail(UW_EINVAL, "NULL argument");
    uw_status st = check_header(h, h->total_bytes);
    if (st != UW_OK) return st;
    if (!aligned(d_direct, 16) || !aligned(d_w, 16)) return fail(UW_EINVAL, "device pointers must be 16-byte aligned");
    GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.wplane = d_direct;
    g.N = h->N;
    g.K = h->K;
    ValueOrder vo;
    value_order(h, &vo);
    std::memcpy(g.vpal, vo.sorted, 16);
    g.base4 = vo.sorted[0] * 0x01010101u;
    const uint64_t T = static_cast<uint64_t>((h->N + 15) / 16), G = static_cast<uint64_t>(h->K / 64);
    g.tiles = static_cast<uint32_t>(T);
    g.dmeta = d_direct + 1536 * T * G;
    g.dside = h->n_raw > 0 ? g.dmeta + (8 * T * G + 63) / 64 * 64 : g.dmeta;
    g.raw_max = h->n_raw > 0 ? static_cast<uint32_t>(h->n_raw - 1) : 0;
    if (T * G == 0) return UW_OK;
    const dim3 grid(static_cast<uint32_t>((T * G + 3) / 4));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (vo.contiguous)
        hipLaunchKernelGGL(expand_direct_kernel<true>, grid, dim3(256), 0, s, g, d_w);
    else
        hipLaunchKernelGGL(expand_direct_kernel<false>, grid, dim3(256), 0, s, g, d_w);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(UW_EHIP, "expand launch failed: %s", hipGetErrorString(e));
    return UW_OK;
}

namespace {

uw_status gemm_launch(const uw_gemm_args* p, void* stream, bool y_zeroed, uint16_t* hout, int64_t ldh)
{
    clear_error();
    if (!p || !p->h) return fail(UW_EINVAL, "NULL argument");
    if (p->M < 0) return fail(UW_ESHAPE, "M < 0");
    if (p->M == 0) return UW_OK;
    GemmArgs g;
    bool contig = false;
    int v = 0;
    uw_status st = make_args(p, g, contig, v);
    if (st != UW_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    const Variant& var = kVariants[v];
    if (hout) {
        // the tiled, wide and dma kernels end in store_out; a K split adds partial sums instead
        if (var.kind == 0 || g.kgroups) return fail(UW_EUNSUPPORTED, "no SwiGLU epilogue for this variant or K split");
        if (ldh < g.N || !aligned(hout, 8)) return fail(UW_EINVAL, "h: ldh must be >= N and h 8-byte aligned");
        g.hout = hout;
        g.ldh = ldh;
    }
    // K split: Y is zeroed first (a kernel, not a memset, so the launch can be captured in
    // a graph) and every slice adds its part with fp32 atomics
    if (g.kgroups && !y_zeroed) {
        e = launch_zero_rows(g.y, g.ldy, g.M, g.N, s);
        if (e != hipSuccess) return fail(UW_EHIP, "zeroing Y failed: %s", hipGetErrorString(e));
    }
    switch (p->src) {
    case UW_W_BF16: e = launch_src<UW_W_BF16, false>(g, var, s); break;
    case UW_W_EXP: e = launch_src<UW_W_EXP, false>(g, var, s); break;
    case UW_W_IDX: e = launch_src<UW_W_IDX, false>(g, var, s); break;
    default: e = contig ? launch_src<UW_W_DIRECT, true>(g, var, s) : launch_src<UW_W_DIRECT, false>(g, var, s); break;
    }
    if (e != hipSuccess) return fail(UW_EHIP, "GEMM launch failed: %s", hipGetErrorString(e));
    return UW_OK;
}

}  // namespace

uw_status launch_gemm(const uw_gemm_args* p, void* stream, bool y_zeroed)
{
    return gemm_launch(p, stream, y_zeroed, nullptr, 0);
}

uw_status launch_gemm_swiglu(const uw_gemm_args* p, uint16_t* h, int64_t ldh, void* stream)
{
    return gemm_launch(p, stream, false, h, ldh);
}

}  // namespace uw

extern "C" {

uw_status uw_recon_gemm(const uw_gemm_args* args, void* stream) { return uw::launch_gemm(args, stream); }

uw_status uw_expand_direct(const uw_header* h, const uint8_t* d_direct, uint16_t* d_w, void* stream)
{
    return uw::launch_expand_direct(h, d_direct, d_w, stream);
}

uw_status uw_recon_gemm_gate_up(const uw_gemm_args* gate, const uw_gemm_args* up, uint16_t* d_h, int64_t ldh,
                                void* stream)
{
    return uw::launch_gate_up_gemm(gate, up, d_h, ldh, stream);
}

int uw_variant_count(void) { return uw::kNumVariants; }

int uw_split_count(int variant, int64_t N, int64_t K, int64_t M, int32_t split_k)
{
    if (K < 64 || K % 64 || N < 1 || M < 0 || split_k < 0 || split_k > K / 64 || variant >= uw::kNumVariants) return 0;
    const int v = variant < 0 ? uw::default_variant(N, K, M, UW_W_DIRECT) : variant;
    return static_cast<int>(uw::resolve_split(uw::kVariants[v], N, K, M, split_k));
}

const char* uw_variant_name(int variant)
{
    if (variant < 0 || variant >= uw::kNumVariants) return "";
    return uw::kVariants[variant].name;
}

int uw_variant_supports(int variant, int64_t N, int64_t K, int64_t M, int32_t src)
{
    if (variant < 0 || variant >= uw::kNumVariants || K % 64 || K < 64) return 0;
    const uw::Variant& v = uw::kVariants[variant];
    // a "ks" variant exists only where it cuts K (elsewhere it would be its unsplit neighbour)
    if (v.kind == 0 && v.ks && uw::skinny_slices(N, K, v.rt) < 2) return 0;
    if (v.kind == 0 && v.xt == 2 && src != UW_W_DIRECT) return 0;  // X by LDS DMA: built for direct planes only
    if (v.kind == 3) return src == UW_W_BF16 && M >= 1 && 2 * N * K < (int64_t{1} << 32) && 2 * M * K < (int64_t{1} << 32);
    if (v.kind == 0) return M >= 1 && M <= (v.rt == 2 && v.nw == 8 && !v.xnear ? 32 : 64);  // rt2 w8 spills beyond 32 rows of X
    return M >= 1;
}

}  // extern "C"
