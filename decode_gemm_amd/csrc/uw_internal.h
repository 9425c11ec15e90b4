// Internal declarations shared by the translation units of libuw.
#pragma once

#include <cstddef>
#include <cstdint>

#include "uw.h"

namespace uw {

// Thread-local error text behind uw_last_error().
void clear_error();
uw_status fail(uw_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Canonical-code tables derived from a header's code lengths: for every length l,
// count[l] codes starting at first_code[l]; their symbols are sorted[first_index[l] ..].
struct CanonTables {
    uint32_t first_code[16];
    uint32_t count[16];
    uint32_t first_index[16];
    uint8_t sorted[16];
    uint32_t n_used;
};
void canon_tables(const uw_header* h, CanonTables* t);

// The palette sorted by exponent value: sorted[v] = v-th smallest palette exponent,
// order[i] = position of palette[i] in that order; contiguous = the n_pal values are
// consecutive integers (then exponent = sorted[0] + position).
struct ValueOrder {
    uint8_t sorted[16];
    uint8_t order[16];
    bool contiguous;
};
void value_order(const uw_header* h, ValueOrder* v);

// Header-level checks shared by uw_inspect / uw_validate_header.
uw_status check_header(const uw_header* h, size_t blob_bytes);

// Expected section layout for given sizes (the same formula the encoder writes).
struct Layout {
    uint64_t off_sm, off_bitmap, off_rowbase, off_raw, off_chunk, off_stream, bytes_stream, total;
};
Layout layout_for(int64_t N, int64_t K, int64_t n_raw, int64_t n_chunks, uint64_t total_bits);

constexpr uint32_t kMagic = 0x31545755u;  // "UWT1"
constexpr uint32_t kDefaultChunk = 256;
constexpr uint32_t kDefaultLmax = 12;
constexpr uint64_t kSectionAlign = 256;
constexpr uint64_t kStreamSlack = 64;

// Device-side launchers (uw_decode.hip, uw_gemm.hip).
enum DecodeMode { DEC_FULL = 0, DEC_EXP = 1, DEC_IDX = 2, DEC_DIRECT = 3 };
constexpr int kPipelines = 5;  // uw_pipeline values 0 .. kPipelines - 1
uw_status launch_decode(const uw_header* h, const void* d_blob, void* d_out, int mode, uint32_t* d_err,
                        void* stream);
// y_zeroed: the caller has already cleared Y (a K-split launch then skips its own clearing)
uw_status launch_gemm(const uw_gemm_args* a, void* stream, bool y_zeroed = false);
// The up projection's GEMM with the SwiGLU in its epilogue: a->d_y holds the gate
// projection's fp32 output (read only, leading dimension a->ldy) and the launch writes
// h[m][n] = bf16(silu(gate) up) (leading dimension ldh, 8-byte aligned), the same bits as
// the GEMM into Y followed by the separate activation kernel. UW_EUNSUPPORTED when the
// variant (skinny) or a K split leaves no such epilogue; the caller then runs the two steps.
uw_status launch_gemm_swiglu(const uw_gemm_args* a, uint16_t* h, int64_t ldh, void* stream);
// An fp32 buffer Y[M][ld] (first N columns) that a fused gate/up launch clears on the way, for
// the K-split launch that follows it on the same stream (16-byte aligned, ld a multiple of 4).
struct ZeroTarget {
    float* y;
    int64_t ld, M, N;
};
uw_status launch_gate_up_gemm(const uw_gemm_args* gate, const uw_gemm_args* up, uint16_t* d_h, int64_t ldh,
                              void* stream, const ZeroTarget* clear = nullptr);
int default_variant(int64_t N, int64_t K, int64_t M, int32_t src);
uint32_t cu_count();  // compute units of the current device
uint32_t stream_cu_count(void* stream);  // compute units a hipStream_t may use (its CU mask)
uint64_t direct_plane_bytes(const uw_header* h);

bool aligned(const void* p, size_t a);

}  // namespace uw
