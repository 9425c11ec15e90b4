// Device helpers that rebuild bf16 weights from the compressed planes (the consumer side
// of the reconstructive matmul in the Unweight blog post, "How the reconstructive matmul
// works": combine the exponent with the sign/mantissa byte and hand the result to the
// matrix units).
//
// A bf16 weight is sign<<15 | exponent<<7 | mantissa; the sign/mantissa plane stores
// sign<<7 | mantissa per weight. Two weights are rebuilt per 32-bit register (the packed
// bf16 pair an MFMA operand holds) with byte permutes, so no per-element branch or shift
// chain is needed. All helpers work on 8 consecutive weights = one 16-byte MFMA operand
// piece.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace uw {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Weights 2t and 2t+1 (t = 0..3 inside an 8-weight piece) from exponent bytes laid out
// as ea = [e0, e2, e4, e6] and eb = [e1, e3, e5, e7] and the sign/mantissa dword that
// holds their bytes.
template <int T>
__device__ __forceinline__ uint32_t pair_from_split(uint32_t ea, uint32_t eb, uint32_t sm)
{
    constexpr uint32_t esel = 0x0C000C00u | T | ((4 + T) << 16);       // [ea_t, 0, eb_t, 0]
    constexpr uint32_t ssel = (T & 1) ? 0x03030202u : 0x01010000u;      // [s, s, s', s']
    const uint32_t ex = __builtin_amdgcn_perm(eb, ea, esel);
    const uint32_t sx = __builtin_amdgcn_perm(sm, sm, ssel) & 0x807F807Fu;
    return (ex << 7) | sx;
}

// Per byte: 0xFF where bit 7 of that byte of v is set, else 0x00 (v_perm's sign-replicate
// selectors 8..11 read bits 15 / 31 of each source dword).
__device__ __forceinline__ uint32_t byte_mask_bit7(uint32_t v)
{
    return __builtin_amdgcn_perm(v, v << 8, 0x0B090A08u);
}

// Exponent bytes for four 4-bit palette indices held one per byte (values 0..15):
// two 8-entry byte lookups (palette bytes 0..7 and 8..15) merged on bit 3.
__device__ __forceinline__ uint32_t palette_lookup(uint32_t sel3, uint32_t hi_mask, const uint32_t* pal)
{
    const uint32_t lo = __builtin_amdgcn_perm(pal[1], pal[0], sel3);
    const uint32_t hi = __builtin_amdgcn_perm(pal[3], pal[2], sel3);
    return (hi & hi_mask) | (lo & ~hi_mask);
}

// Split an index dword (8 nibbles: weight 2u in the low nibble of byte u, 2u+1 in the
// high nibble) into the exponent bytes of the even and the odd weights.
__device__ __forceinline__ void exps_from_idx(uint32_t idx, const uint32_t* pal, uint32_t& ea, uint32_t& eb)
{
    ea = palette_lookup(idx & 0x07070707u, byte_mask_bit7(idx << 4), pal);
    eb = palette_lookup((idx >> 4) & 0x07070707u, byte_mask_bit7(idx), pal);
}

// Same split for 8 exponent bytes given in natural order (e0..e3, e4..e7).
__device__ __forceinline__ void split_exps(uint32_t e_lo, uint32_t e_hi, uint32_t& ea, uint32_t& eb)
{
    ea = __builtin_amdgcn_perm(e_hi, e_lo, 0x06040200u);
    eb = __builtin_amdgcn_perm(e_hi, e_lo, 0x07050301u);
}

// 8 bf16 weights from split exponents and the two sign/mantissa dwords.
__device__ __forceinline__ u32x4 piece_from_split(uint32_t ea, uint32_t eb, uint32_t sm_lo, uint32_t sm_hi)
{
    u32x4 r;
    r.x = pair_from_split<0>(ea, eb, sm_lo);
    r.y = pair_from_split<1>(ea, eb, sm_lo);
    r.z = pair_from_split<2>(ea, eb, sm_hi);
    r.w = pair_from_split<3>(ea, eb, sm_hi);
    return r;
}

// ---- direct plane (see uw_prepare_direct): per 8-weight unit, one index dword whose
// byte b holds weight b (low nibble) and weight b+4 (high nibble), and two dwords of
// rearranged sign/mantissa bytes (mantissa << 1 | sign of the pair partner).

// Two bf16 weights from [sm'_a, e_a, sm'_b, e_b]: rotating right by one bit moves each
// mantissa into bits 0..6 / 16..22, each exponent into bits 7..14 / 23..30, and each
// partner-sign bit into the other half's sign position.
__device__ __forceinline__ uint32_t rotr1(uint32_t v) { return __builtin_rotateright32(v, 1); }

// Exponent bytes [e0, e1, e2, e3] (lo) and [e4..e7] (hi) of one unit. CONTIG: the
// value-sorted palette is a run of consecutive exponents starting at base (base4 =
// base * 0x01010101), so exponent = base + index, a byte-wise add with no carries.
// Otherwise two 8-entry byte lookups in the value-sorted palette vpal.
template <bool CONTIG>
__device__ __forceinline__ void unit_exps(uint32_t idx, uint32_t base4, const uint32_t* vpal, uint32_t& lo, uint32_t& hi)
{
    const uint32_t x = idx & 0x0F0F0F0Fu, y = (idx >> 4) & 0x0F0F0F0Fu;
    if (CONTIG) {
        lo = x + base4;
        hi = y + base4;
    } else {
        lo = palette_lookup(x & 0x07070707u, byte_mask_bit7(x << 4), vpal);
        hi = palette_lookup(y & 0x07070707u, byte_mask_bit7(y << 4), vpal);
    }
}

// 8 bf16 weights (one MFMA operand piece) of a unit from its exponent dwords (natural
// order) and its two sign/mantissa dwords.
__device__ __forceinline__ u32x4 unit_piece(uint32_t e_lo, uint32_t e_hi, uint32_t s_lo, uint32_t s_hi)
{
    u32x4 r;
    r.x = rotr1(__builtin_amdgcn_perm(e_lo, s_lo, 0x05010400u));  // [s0, e0, s1, e1]
    r.y = rotr1(__builtin_amdgcn_perm(e_lo, s_lo, 0x07030602u));  // [s2, e2, s3, e3]
    r.z = rotr1(__builtin_amdgcn_perm(e_hi, s_hi, 0x05010400u));
    r.w = rotr1(__builtin_amdgcn_perm(e_hi, s_hi, 0x07030602u));
    return r;
}

// ---- SwiGLU (the glue between gate/up and down in the MLP): h = bf16(silu(g) * u), one
// rounding to nearest even from fp32. Shared by the stand-alone kernel and the fused
// gate/up epilogue so that both give the same bits.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN -> quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace uw
