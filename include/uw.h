/*
 * uw.h -- C ABI of libuw: lossless bf16 weight compression by exponent coding, with
 * GPU decoders and a reconstructive GEMM for AMD Instinct MI355X (gfx950).
 *
 * The method is the one Cloudflare describes in "Unweight: how we compressed an LLM
 * 22% without sacrificing quality":
 *   - a bf16 weight is sign (1 bit), exponent (8 bits), mantissa (7 bits); sign and
 *     mantissa are kept verbatim ("How weights compress");
 *   - the exponent byte is replaced by an index into the 16 most common exponents of
 *     the matrix and Huffman-coded; a 64-weight row holding any exponent outside
 *     those 16 is stored as-is ("Exponents are predictable");
 *   - four execution pipelines consume it: full decode + plain GEMM, exponent-only
 *     decode, runtime palette transcode, and direct palette prepared at load ("Four
 *     ways to use compressed weights");
 *   - three of them use a reconstructive matmul that rebuilds bf16 tiles on chip and
 *     feeds them to the matrix units, so the rebuilt weights never reach HBM ("How the
 *     reconstructive matmul works");
 *   - an autotuner picks the pipeline per matrix and batch size by measurement ("Why
 *     no single pipeline wins").
 *
 * Conventions for every entry point:
 *   - Weights W are [N][K] row-major bf16 bit patterns (PyTorch Linear layout: N = out
 *     features, K = in features). K must be a multiple of 64. X is [M][K] bf16 row-major
 *     with leading dimension ldx; Y = X * W^T is [M][N] fp32 with leading dimension ldy.
 *   - "d_" pointers are device (HBM) pointers; all others are host pointers.
 *   - The caller owns every buffer. The library never allocates or frees device memory
 *     and keeps no pointer after a call returns. Every kernel is the library's own; it
 *     links no vendor math library.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Device
 *     calls are asynchronous on that stream; their return value reports argument
 *     validation and launch errors only.
 *   - No C++ exception crosses this boundary. On failure a status code is returned and
 *     a thread-local message is available from uw_last_error().
 *   - All functions are re-entrant. The only global state is a once-per-process flag per
 *     kernel recording that its LDS-size attribute has been raised.
 */
#ifndef UW_H
#define UW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UW_VERSION 1

/* Status codes. */
typedef enum {
    UW_OK = 0,
    UW_EINVAL = 1,       /* bad argument: NULL / misaligned pointer, bad option, bad ld */
    UW_ESHAPE = 2,       /* bad shape: N < 1, K < 1, K % 64 != 0, M < 0 */
    UW_EFORMAT = 3,      /* blob fails validation (magic, version, sizes, offsets) */
    UW_ERANGE = 4,       /* value out of the format's range (stream bits >= 2^32, ...) */
    UW_ENOSPACE = 5,     /* output / workspace buffer too small; required size returned */
    UW_EHIP = 6,         /* a HIP runtime call or kernel launch failed */
    UW_EUNSUPPORTED = 7, /* combination not supported by this build */
    UW_EINTERNAL = 8     /* unexpected internal failure */
} uw_status;

/* Static string naming a status code. Never NULL. */
const char* uw_status_string(int status);
/* Thread-local description of the last failure in this thread ("" if none). */
const char* uw_last_error(void);
/* UW_VERSION of the built library. */
int uw_version(void);

/*
 * Blob header: the first 256 bytes of every blob, byte for byte (little-endian).
 * Blob layout (format version 1): header, then these sections, each starting at a
 * multiple of 256 bytes:
 *   sm       [N*K]   u8   sign<<7 | mantissa of every weight, row-major
 *   bitmap   [N*bitmap_words] u32  bit (j%32) of word (n*bitmap_words + j/32) set iff the
 *                         64-weight group W[n][64j .. 64j+63] is raw
 *   row_base [N+1]   u32  number of raw groups in rows before n
 *   raw      [n_raw][64] u8  verbatim exponent bytes of every raw group, (n, j) order
 *   chunk    [n_chunks+1] u32  chunk c covers flattened elements [c*chunk, (c+1)*chunk);
 *                         entry c = stream bits of all symbols before chunk c
 *   stream   [bytes_stream] u8  canonical Huffman codes of the palette index of every
 *                         element of a non-raw group, row-major order, MSB first; stream
 *                         bit b is bit 31-(b%32) of little-endian u32 word b/32; zero
 *                         padded, with at least 64 bytes of zero slack after the last bit
 * Palette: the min(16, #distinct) most frequent exponent bytes of the matrix, by count
 * descending then value ascending; palette index = rank. code_len[i] = code length of
 * index i (0 = index unused in the stream). Codes are canonical (RFC 1951 3.2.2 rule).
 */
typedef struct uw_header {
    uint32_t magic;   /* 0x31545755, the bytes "UWT1" */
    uint32_t version; /* 1 */
    int64_t N, K;
    uint32_t chunk;    /* elements per chunk, a multiple of 64 */
    uint32_t lmax;     /* longest allowed code, 1..15 */
    uint32_t n_pal;    /* palette entries, 0..16 */
    uint32_t n_chunks; /* ceil(N*K / chunk) */
    uint8_t palette[16];
    uint8_t code_len[16];
    int64_t n_raw;       /* raw 64-weight groups */
    uint64_t total_bits; /* stream bits, < 2^32 */
    uint64_t off_sm, off_bitmap, off_rowbase, off_raw, off_chunk, off_stream;
    uint64_t bytes_stream; /* stream section bytes including padding and slack */
    uint64_t total_bytes;  /* whole blob */
    uint32_t bitmap_words; /* ceil(K / 2048) */
    uint32_t reserved[25]; /* zero */
} uw_header;

typedef struct {
    uint32_t chunk; /* elements per chunk, multiple of 64; 0 = default (256) */
    uint32_t lmax;  /* 1..15; 0 = default (12) */
} uw_encode_opts;

/*
 * uw_encode (host). Compress W (host, [N][K] bf16 bits) into a self-describing blob
 * ("How weights compress", "Exponents are predictable"). Two-call size query: if blob
 * is NULL or *blob_bytes is smaller than required, returns UW_ENOSPACE and sets
 * *blob_bytes to the required size; on success *blob_bytes = bytes written. opts may be
 * NULL (defaults). Errors: UW_ESHAPE (N < 1, K < 1, K % 64), UW_EINVAL (NULL w or
 * blob_bytes, chunk not a multiple of 64, lmax outside 1..15 or too small for the number
 * of used palette indices), UW_ERANGE (stream would need >= 2^32 bits, or more than 2^32
 * raw groups).
 */
uw_status uw_encode(const uint16_t* w_bf16, int64_t N, int64_t K, const uw_encode_opts* opts, void* blob,
                    size_t* blob_bytes);

/* uw_inspect (host). Validate a blob held in host memory (header fields, section
 * offsets and sizes, chunk offsets monotone and ending at total_bits, row_base
 * consistent with the bitmap) and copy its header to *out. UW_EFORMAT on any
 * inconsistency, UW_EINVAL on NULL arguments. */
uw_status uw_inspect(const void* blob, size_t blob_bytes, uw_header* out);

/* uw_validate_header (host). The header-only subset of uw_inspect, for a blob already
 * on the device: checks the header's own fields, its section offsets and
 * total_bytes <= blob_bytes. */
uw_status uw_validate_header(const uw_header* h, size_t blob_bytes);

/*
 * Device decoders ("Four ways to use compressed weights"; the Huffman decoder and
 * palette transcoder of "Sharing the GPU between decode and compute").
 *   h       host copy of the blob's header (from uw_inspect / uw_validate_header)
 *   d_blob  the blob, copied verbatim to device memory, 256-byte aligned
 *   d_err   optional device u32: kernels OR in UW_DERR_* bits on corrupt input; the
 *           caller clears it. NULL = no reporting (output is then undefined on corrupt
 *           input, but every access stays inside the blob).
 * Outputs (device, 16-byte aligned, caller-owned):
 *   uw_decode_full:       d_w   [N][K] bf16 bits (2 bytes / weight), bit-exact W
 *   uw_decode_exponent:   d_exp [N][K] u8 exponent bytes, raw groups included (1 B/w)
 *   uw_transcode_palette: d_idx [N*K/2] u8, element i in the low nibble of byte i/2 when
 *                         i is even, the high nibble when odd; raw groups hold 0 (0.5 B/w)
 */
#define UW_DERR_BADCODE 1u    /* a bit pattern that is no code of the table */
#define UW_DERR_CHUNKLEN 2u   /* a chunk's symbols did not end at the next chunk offset */
#define UW_DERR_RAWINDEX 4u   /* uw_prepare_direct: the bitmap / row_base place a raw group
                                 at or past the header's n_raw (that row is left out of its
                                 block's raw mask; nothing is written outside the plane) */
uw_status uw_decode_full(const uw_header* h, const void* d_blob, uint16_t* d_w, uint32_t* d_err, void* stream);
uw_status uw_decode_exponent(const uw_header* h, const void* d_blob, uint8_t* d_exp, uint32_t* d_err, void* stream);
uw_status uw_transcode_palette(const uw_header* h, const void* d_blob, uint8_t* d_idx, uint32_t* d_err,
                               void* stream);

/*
 * uw_prepare_direct (device). The load-time preparation of the direct-palette pipeline
 * ("Four ways to use compressed weights": weights are transcoded once at model load
 * into a compact 4-bit palette form that the matmul consumes with no per-call
 * preprocessing). Decodes the Huffman stream into the direct plane d_direct
 * (uw_direct_plane_bytes, 16-byte aligned), laid out for the reconstructive GEMM's
 * operand registers. With T = ceil(N/16) row tiles and G = K/64 groups:
 *   blocks  T*G blocks of 1536 bytes, group-major: block (t, j) at 1536*(j*T + t), so
 *           the blocks of one 64-weight group are adjacent for all row tiles. Lane l = 16*g + r
 *           (g = 0..3, r = 0..15) of the MFMA operand owns row 16t+r, weights
 *           64j+16g .. 64j+16g+15:
 *             bytes 16l .. 16l+15    weight x: (mantissa_x << 1) | sign of weight x^1
 *                                    (each byte keeps its own mantissa and its pair
 *                                    partner's sign, so two bf16 weights are one byte
 *                                    permute and one rotate)
 *             bytes 1024+8l .. +7    two index dwords, one per 8-weight unit; byte b of
 *                                    a unit dword holds unit weight b in its low nibble
 *                                    and weight b+4 in its high nibble
 *           The index is the position of the weight's exponent in the palette sorted by
 *           exponent value (ascending); in a raw group it is 0 and the sign/mantissa
 *           bytes are still those of the weights. Rows >= N are zero.
 *   meta    at 1536*T*G: per block, at 8*(t*G + j) (tile-major: a row tile's metas are
 *           adjacent), two u32: a mask whose bit r says row 16t+r's group j is raw, and the
 *           side-table index of the block's first raw row.
 *   side    at 1536*T*G + round_up(8*T*G, 64) (the bytes in between are zero): 64
 *           exponent bytes per raw (row, group), ordered by tile, then group, then row.
 * A wave therefore reads one contiguous kilobyte per operand load, a small-batch GEMM whose
 * workgroups step through the groups together reads one contiguous region of the plane at
 * a time, and a raw row only swaps in its verbatim exponents. d_err as for the decoders.
 */
uw_status uw_prepare_direct(const uw_header* h, const void* d_blob, uint8_t* d_direct, uint32_t* d_err, void* stream);
/*
 * uw_expand_direct (device). The bf16 weights W[N][K] (row-major, bit patterns) written to
 * d_w from a direct plane made by uw_prepare_direct: the full decode of "Four ways to use
 * compressed weights" (original weights rebuilt in HBM for a plain GEMM), fed from the
 * load-time palette plane instead of the Huffman stream, so it is a pure streaming kernel
 * (reads ~1.52 bytes per weight, writes 2). The result is bit-identical to uw_decode_full
 * of the blob the plane was made from. d_direct, d_w: device, 16-byte aligned; d_w holds
 * 2*N*K bytes. Errors: UW_EINVAL (NULL or misaligned pointers), UW_EFORMAT (bad header),
 * UW_EHIP.
 */
uw_status uw_expand_direct(const uw_header* h, const uint8_t* d_direct, uint16_t* d_w, void* stream);
/* Bytes of the direct plane of a blob: 1536*T*G + round_up(8*T*G, 64) + 64*n_raw. */
uw_status uw_direct_plane_bytes(const uw_header* h, size_t* out);

/*
 * uw_recon_gemm (device). Y = X * W^T with W taken from one of three planes ("How the
 * reconstructive matmul works"): the bf16 weights themselves (plain GEMM of the
 * full-decode pipeline), the exponent plane plus the blob's sign/mantissa plane, or the
 * 4-bit palette-index plane plus the sign/mantissa plane, the palette and the raw
 * groups. Weights are rebuilt in registers / LDS and fed to bf16 MFMA; they are never
 * written to memory. Accumulation is fp32; Y is overwritten (not accumulated into).
 * K split: every variant can cut K into slices of whole 64-groups, one workgroup per
 * (output tile, slice); Y is then zeroed on the stream and each slice adds its partial
 * sums into Y with fp32 atomics. split_k = 0 takes the variant's own choice: the 128x128
 * and 256x256 tiles and the skinny variants named "... ks" split when a problem has too
 * few output tiles to fill the GPU (long K, small N*M), the others do not; split_k = s >= 1
 * asks for s slices (rounded so that every slice has the same whole number of groups;
 * uw_split_count gives the count a launch will use). With three or more slices the order
 * of the additions is not fixed, so Y may differ in the last bits from run to run (always
 * within the same error bound); one or two slices give identical results. The default
 * variant (-1) never picks a "ks" variant, and uw_variant_supports reports one only for
 * shapes it actually splits.
 */
typedef enum { UW_W_BF16 = 0, UW_W_EXP = 1, UW_W_IDX = 2, UW_W_DIRECT = 3 } uw_wsrc;

typedef struct {
    int64_t M;             /* rows of X and Y; 0 is a no-op */
    const uint16_t* d_x;   /* X bf16 [M][ldx], 16-byte aligned */
    int64_t ldx;           /* >= K, multiple of 8 */
    const uw_header* h;    /* N, K, palette */
    const void* d_blob;    /* device blob (sm plane, raw tables); unused for UW_W_BF16 */
    int32_t src;           /* uw_wsrc */
    const void* d_wplane;  /* bf16 W [N][K] | exponent plane [N][K] | index plane [N*K/2] |
                              direct plane (uw_prepare_direct) */
    float* d_y;            /* Y fp32 [M][ldy], 16-byte aligned */
    int64_t ldy;           /* >= N */
    int32_t variant;       /* kernel variant id, -1 = default for (N, K, M) */
    int32_t split_k;       /* K slices, 0 = the variant's choice, 1..K/64 (see above) */
} uw_gemm_args;

uw_status uw_recon_gemm(const uw_gemm_args* args, void* stream);

/* uw_split_count (host): the number of K slices a launch of `variant` (-1 = default) with
 * split_k uses on (N, K, M); 0 when the arguments are invalid (split_k < 0 or > K/64, an
 * unknown variant, K not a positive multiple of 64). */
int uw_split_count(int variant, int64_t N, int64_t K, int64_t M, int32_t split_k);

/*
 * uw_recon_gemm_gate_up (device). The gate and up projections of a SwiGLU MLP and the
 * SwiGLU itself in one launch (the small-batch fixed cost the post lists among the
 * reconstructive matmul's overheads, "Bundles and results" / "Trade-offs": one launch for
 * gate and up). gate and up are two uw_gemm_args as for uw_recon_gemm, both on the
 * direct plane (src UW_W_DIRECT) with the same M (1..64), N, K and X (d_x, ldx); each
 * block streams its rows of gate and the same rows of up through one load ring, with
 * gate's GEMM variant: 4-wave variants take a K group of both matrices per step (each X
 * group fetched once for the two), 8-wave variants all of gate's groups, then up's. A
 * variant with 8 waves and X rings ("xd") has no fused form past M = 32. Writes gate->d_y and
 * up->d_y (fp32, exactly what uw_recon_gemm gives with that variant) and
 * d_h[M][ldh] = bf16(silu(gate) * up), the same bits as uw_swiglu on those outputs.
 * Errors: UW_EINVAL / UW_ESHAPE as for uw_recon_gemm (UW_EINVAL also when gate and up
 * name different X), and UW_EUNSUPPORTED when the fused
 * form does not apply (not both direct planes, M > 64, a palette whose exponents are not
 * consecutive, a variant without a fused form, or a K split); the caller then runs the
 * two GEMMs and uw_swiglu.
 */
uw_status uw_recon_gemm_gate_up(const uw_gemm_args* gate, const uw_gemm_args* up, uint16_t* d_h, int64_t ldh,
                                void* stream);

/* Kernel variants of uw_recon_gemm (tile shape per CU and pipelining depth, "How the
 * reconstructive matmul works": wider tiles for large batches, deeper buffers for small
 * ones). uw_variant_count() variants exist; uw_variant_name() describes one;
 * uw_variant_supports() says whether a variant accepts (N, K, M, src). The variants take
 * every src with two exceptions, so the plain bf16 GEMM of the full-decode pipeline ("Four
 * ways to use compressed weights": the decoded weights go to a standard matrix multiply) is
 * the same kernel family on the UW_W_BF16 loader: the skinny "... xd" variants (X by LDS DMA)
 * take direct planes only, and the "dma ..." variants (both operands sent from memory straight
 * into LDS, no rebuild step: a 256x256 tile through two stages, or 256x128 through three) take
 * UW_W_BF16 only, with X and W each under 4 GiB. */
int uw_variant_count(void);
const char* uw_variant_name(int variant);
int uw_variant_supports(int variant, int64_t N, int64_t K, int64_t M, int32_t src);

/*
 * Pipelines ("Four ways to use compressed weights"):
 *   UW_PIPE_FULL      uw_decode_full into workspace, then plain bf16 GEMM
 *   UW_PIPE_EXP       uw_decode_exponent into workspace, then reconstructive GEMM
 *   UW_PIPE_TRANSCODE uw_transcode_palette into workspace, then reconstructive GEMM
 *   UW_PIPE_DIRECT    reconstructive GEMM on the direct plane prepared once at load
 *                     (uw_prepare_direct)
 *   UW_PIPE_EXPAND    uw_expand_direct of that direct plane into workspace, then plain
 *                     bf16 GEMM: the full-decode pipeline fed from the load-time plane
 *                     (a streaming kernel) instead of the Huffman stream, for batches
 *                     large enough that the plain bf16 GEMM beats the reconstructive one
 */
typedef enum {
    UW_PIPE_FULL = 0,
    UW_PIPE_EXP = 1,
    UW_PIPE_TRANSCODE = 2,
    UW_PIPE_DIRECT = 3,
    UW_PIPE_EXPAND = 4
} uw_pipeline;

/* A per-(matrix, M) execution plan: which pipeline, GEMM variant and K split ("Why no
 * single pipeline wins": the per-model profile). t_ms = measured time per forward. */
typedef struct {
    int32_t pipeline;
    int32_t variant;
    float t_ms;
    int32_t split_k; /* the slice count measured (as uw_split_count reports it) */
} uw_plan;

/* Workspace bytes a pipeline needs for a matrix (the preprocessing slot: 2, 1, 0.5, 0 or
 * 2 bytes per weight for full / exp / transcode / direct / expand). */
uw_status uw_workspace_bytes(const uw_header* h, int32_t pipeline, size_t* out);

/* Run one pipeline end to end on `stream`: decode into d_ws if the pipeline needs it,
 * then the GEMM with `variant` and `split_k` (as in uw_gemm_args). d_direct = the direct
 * plane from uw_prepare_direct (UW_PIPE_DIRECT and UW_PIPE_EXPAND only). */
uw_status uw_run_pipeline(int32_t pipeline, int32_t variant, int32_t split_k, const uw_header* h, const void* d_blob,
                          const uint8_t* d_direct, int64_t M, const uint16_t* d_x, int64_t ldx, float* d_y,
                          int64_t ldy, void* d_ws, size_t ws_bytes, uint32_t* d_err, void* stream);

/*
 * uw_run_pipeline_noalloc (device). uw_run_pipeline for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels, with the preprocessing slot taken from a scratch array
 * the library holds in device memory, uw_noalloc_scratch_bytes() bytes (128 MiB) per GPU,
 * from the library's load until the process ends. No device memory is allocated or freed
 * by the call; the first call on a device looks the array's address up. The caller still
 * passes X, Y, the blob and the direct plane. Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (on different streams, or from several threads)
 * race on it and must be ordered by the caller. Errors: those of uw_run_pipeline, and
 * UW_ENOSPACE when the pipeline's slot (uw_workspace_bytes) exceeds the array.
 */
uw_status uw_run_pipeline_noalloc(int32_t pipeline, int32_t variant, int32_t split_k, const uw_header* h,
                                  const void* d_blob, const uint8_t* d_direct, int64_t M, const uint16_t* d_x,
                                  int64_t ldx, float* d_y, int64_t ldy, uint32_t* d_err, void* stream);
/* Bytes of the scratch array behind uw_run_pipeline_noalloc (the largest slot it takes). */
size_t uw_noalloc_scratch_bytes(void);

/* One projection of a model and how it runs: its header and device blob, its direct plane
 * (uw_prepare_direct) or NULL, and its plan (pipeline, GEMM variant, K split). Used by the
 * autotuner's rotation set and by the MLP stack below. */
typedef struct {
    const uw_header* h;       /* the projection's header (host) */
    const void* d_blob;       /* its blob on the device */
    const uint8_t* d_direct;  /* its direct plane; required for UW_PIPE_DIRECT and UW_PIPE_EXPAND */
    int32_t pipeline;         /* uw_pipeline */
    int32_t variant;          /* GEMM variant, -1 = default */
    int32_t split_k;          /* K split, 0 = the variant's choice */
} uw_proj;

/*
 * uw_autotune (device, synchronous). For each M in Ms, time every supported (pipeline,
 * variant, K split) candidate and return the fastest in out[i] ("Why no single pipeline
 * wins", "Sharing the GPU between decode and compute": measured, not heuristic).
 *
 * A candidate is timed the way a plan runs in a model: `reps` forwards launched back to
 * back on `stream`, cycling through the rotation set (rot[0 .. n_rot-1]: matrices of the
 * same N and K, e.g. the same projection of successive layers or copies of one matrix,
 * so that caches hold none of the weights), between two HIP events; that is repeated
 * `trials` times after `warmup` untimed forwards, and t_ms is the median over the trials
 * of the mean time per forward. Without a rotation set (rot NULL or n_rot 0) the single
 * matrix (h, d_blob, d_direct) is used. With tune_split, every candidate variant is also
 * timed at the K splits 1, 2, 3, 4, 6, 8 (those that keep at least 8 groups per slice
 * and that differ from each other), besides its own choice; otherwise only its own choice.
 *
 * Direct-palette and expand candidates need a direct plane for every matrix of the set;
 * pipeline_mask 0 means every pipeline (bits 0..4). d_x must hold max(Ms) rows of K bf16,
 * d_y max(Ms) rows of N fp32, and d_ws at least the largest uw_workspace_bytes of the
 * candidate pipelines (smaller workspaces drop the pipelines that do not fit). Blocks
 * until the measurements finish. Errors: UW_EINVAL (arguments, a rotation entry of
 * another shape), UW_EUNSUPPORTED (no candidate for some M), UW_EHIP.
 */
typedef struct {
    const uw_header* h;      /* shape (N, K); the matrix timed when there is no rotation set */
    const void* d_blob;
    const uint8_t* d_direct; /* direct plane (uw_prepare_direct) or NULL */
    const uint16_t* d_x;  /* [max M][K] bf16 */
    float* d_y;           /* [max M][N] fp32 */
    void* d_ws;
    size_t ws_bytes;
    int32_t reps;   /* forwards per trial, >= 1 (0 = 10) */
    int32_t warmup; /* untimed forwards per candidate (0 = 2) */
    uint32_t pipeline_mask; /* bit p set = pipeline p is a candidate (0 = all) */
    int32_t variant_mask;   /* bit v set = GEMM variant v is a candidate (0 = all) */
    void* d_scrub;          /* optional device buffer overwritten before every trial
                               (outside the timed region); NULL = no scrubbing */
    size_t scrub_bytes;     /* multiple of 16 */
    const uw_proj* rot;     /* rotation set (pipeline / variant fields ignored), or NULL */
    int32_t n_rot;
    int32_t trials;         /* timed trials per candidate (0 = 3) */
    int32_t tune_split;     /* nonzero: also time the K splits listed above */
} uw_tune_args;

uw_status uw_autotune(const uw_tune_args* args, const int64_t* Ms, int nM, void* stream, uw_plan* out);

/*
 * Model bundle (host). One file for distribution and inference ("Bundles and results":
 * every projection Huffman-coded in one package, transcoded at load into the form its
 * pipeline reads, e.g. with uw_prepare_direct), together with the per-model profile of
 * measured plans ("Sharing the GPU between decode and compute": pipeline, matmul variant
 * and K split per projection shape and batch size). All calls work on caller buffers
 * holding the whole bundle in host memory (a read file or a mapping of it).
 *
 * Layout (little-endian, offsets multiples of 256): a 64-byte header ("UWB1", version 1,
 * counts, table offsets, total size, checksum of the tables); n_items records of 128
 * bytes (name, blob offset, blob bytes, blob checksum); n_plans records of 96 bytes (N, K,
 * M, pipeline, split_k, t_ms, variant name); then the blobs verbatim, each 256-byte
 * aligned. Variants are stored by name so that a profile outlives a change of the
 * variant table (uw_variant_by_name maps a name back; -1 when this build lacks it).
 */
#define UW_BUNDLE_NAME_MAX 64
typedef struct {
    const char* name;   /* NUL-terminated, 1..63 bytes, unique in the bundle */
    const void* blob;   /* host blob from uw_encode */
    size_t blob_bytes;
} uw_bundle_item;

typedef struct {
    int64_t N, K;       /* the projection shape the plan is for */
    int64_t M;          /* batch size */
    int32_t pipeline;   /* uw_pipeline */
    int32_t split_k;    /* as in uw_gemm_args */
    float t_ms;         /* measured time per forward */
    char variant[48];   /* uw_variant_name of the GEMM variant, "" = the default */
} uw_bundle_plan;

typedef struct {
    uint32_t n_items, n_plans;
    uint64_t total_bytes;
} uw_bundle_info;

typedef struct {
    char name[UW_BUNDLE_NAME_MAX];
    uint64_t offset;      /* of the blob from the start of the bundle (256-byte aligned) */
    uint64_t blob_bytes;
    uw_header header;     /* the blob's header (header-level checks passed) */
} uw_bundle_entry;

/* uw_bundle_write: write a bundle of n_items blobs (each validated with uw_inspect) and
 * n_plans plans into out. Two-call size query as for uw_encode (out NULL or *out_bytes
 * too small: UW_ENOSPACE with the size needed). Errors: UW_EINVAL (names empty, too long
 * or repeated; a bad plan record), the blob's own validation status. */
uw_status uw_bundle_write(const uw_bundle_item* items, int n_items, const uw_bundle_plan* plans, int n_plans, void* out,
                          size_t* out_bytes);
/* uw_bundle_open: validate a bundle in memory (header, tables and their checksum, every
 * item's place and blob header; with verify != 0 also each blob's checksum and full
 * uw_inspect validation) and report its counts. UW_EFORMAT on any inconsistency. */
uw_status uw_bundle_open(const void* bundle, size_t bytes, int verify, uw_bundle_info* info);
/* Item i (name, where its blob sits, its header) and plan i of a bundle. */
uw_status uw_bundle_item_at(const void* bundle, size_t bytes, uint32_t i, uw_bundle_entry* out);
uw_status uw_bundle_plan_at(const void* bundle, size_t bytes, uint32_t i, uw_bundle_plan* out);
/* Index of the variant named `name`, or -1. */
int uw_variant_by_name(const char* name);

/*
 * uw_swiglu (device). The activation between the MLP projections of a SwiGLU layer:
 * h[i] = bf16(silu(g[i]) * u[i]), silu(z) = z / (1 + e^-z), fp32 math, rounded to
 * nearest-even bf16. g, u fp32 [n], h bf16 [n], all 16-byte aligned.
 */
uw_status uw_swiglu(const float* d_g, const float* d_u, int64_t n, uint16_t* d_h, void* stream);

/*
 * MLP stack (device). One SwiGLU MLP per layer, layers in order: g = X Wg^T, u = X Wu^T,
 * h = bf16(silu(g) u) (uw_swiglu), Y = h Wd^T, each projection through its own pipeline,
 * GEMM variant and K split (e.g. from uw_autotune), all launched on `stream` ("Bundles and
 * results": gate, activation, up and down per layer; "Sharing the GPU between decode and
 * compute": the next matrix is prepared while the current one multiplies).
 *
 * Every layer reads the same X (bf16 [M][K], K = the gate/up input width, 16-byte
 * aligned; attention between layers is not modelled) and overwrites d_y (fp32
 * [M][N_out], N_out = down's N); after the call d_y holds the last layer's output.
 * With decode_stream != NULL the decode-first projections (full / exp / transcode) are
 * decoded on decode_stream into two alternating workspace slots, each one projection ahead
 * of its GEMM; events created by the call order the two streams (the caller's streams keep
 * their own priorities). All layers must have the same shapes: gate and up N_ff x K, down
 * N_out x N_ff. Buffers are the caller's; nothing is allocated on the device.
 *
 * Where the up projection runs a tiled, wide or dma variant in one K slice, the SwiGLU is
 * computed in that GEMM's epilogue (from g and the tile's up outputs, the same bits as
 * uw_swiglu) and u is not stored; elsewhere the up GEMM writes u and uw_swiglu follows.
 *
 * Workspace, uw_mlp_stack_workspace: g and u (fp32 M x N_ff), h (bf16 M x N_ff) and one
 * decode slot (two when two_slots != 0) of the largest plane the layers' pipelines decode,
 * each part 256-byte aligned. After the call g and h hold the last layer's values, and u
 * too unless that layer's up GEMM took the SwiGLU epilogue.
 * Errors: UW_EINVAL (NULL pointers, bad pipeline, direct plane missing), UW_ESHAPE
 * (shapes differ or do not chain), UW_ENOSPACE (workspace too small), UW_EHIP.
 */
typedef struct {
    uw_proj gate, up, down;
} uw_mlp_layer;

uw_status uw_mlp_stack_workspace(const uw_mlp_layer* layers, int n_layers, int64_t M, int two_slots, size_t* out);
uw_status uw_mlp_stack_forward(const uw_mlp_layer* layers, int n_layers, int64_t M, const uint16_t* d_x, float* d_y,
                               void* d_ws, size_t ws_bytes, void* stream, void* decode_stream);

/*
 * Stack schedule options ("Sharing the GPU between decode and compute": hard layers, whose
 * projections need preprocessing, are decoded on a side stream while the layers before them
 * compute, through preprocessing slots; down is consumed last in a layer, so its decode may
 * be issued first).
 *
 * uw_mlp_stack_forward_ex is uw_mlp_stack_forward with:
 *   slots      decode slots in the workspace (1..8; 0 = 2). With decode_stream != NULL the
 *              decode-first projections of all layers, taken in decode order, use slot
 *              q mod slots; after every GEMM that frees a slot, each decode whose slot is free
 *              is issued on decode_stream, so a hard layer is decoded while the easy layers
 *              (all projections direct palette) before it compute. Without a decode stream
 *              only slot 0 is used.
 *   down_first per layer, decode down before gate and up (decode order down, gate, up) instead
 *              of gate, up, down. An order that would need a slot still held by a later GEMM
 *              (down_first with fewer slots than a layer's decode-first projections) is
 *              rejected with UW_EINVAL before anything is launched.
 * Results are bit-identical to uw_mlp_stack_forward for every slot count and order (the
 * same kernels on the same planes). uw_mlp_stack_workspace_ex sizes the workspace for
 * opts->slots slots (uw_mlp_stack_workspace(two_slots) = slots 2 or 1).
 */
typedef struct {
    int32_t slots;
    int32_t down_first;
} uw_stack_opts;

uw_status uw_mlp_stack_workspace_ex(const uw_mlp_layer* layers, int n_layers, int64_t M, const uw_stack_opts* opts,
                                    size_t* out);
uw_status uw_mlp_stack_forward_ex(const uw_mlp_layer* layers, int n_layers, int64_t M, const uint16_t* d_x, float* d_y,
                                  void* d_ws, size_t ws_bytes, void* stream, void* decode_stream,
                                  const uw_stack_opts* opts);

/*
 * uw_mlp_stack_autotune (device, synchronous): coordinate descent over a stack's plan,
 * measured end to end ("Why no single pipeline wins": the configuration space is searched by
 * timing, not by heuristics). Layers fall into two classes: those whose three projections
 * all have direct planes, and the others ("hard" layers, which keep only the Huffman blob
 * for some projection and always need preprocessing). The coordinates are (class, role)
 * for role gate, up, down of each class present, and, with a decode stream and at least 3
 * slots, the decode order. Each pass tries every other pipeline (in pipeline_mask; direct
 * palette and expand only where every layer of the class has that projection's direct
 * plane) for one
 * coordinate at a time, applied to all layers of the class with the default GEMM variant,
 * times the whole forward (warmup untimed runs, then the median of reps, HIP events on
 * `stream`) and keeps a change only if it is at least 1% faster; passes repeat, gate, up,
 * down, until one changes nothing or max_passes is reached.
 *
 * In: layers with blobs, direct planes (or NULL) and a starting plan that runs in the
 * workspace; d_x (M x K bf16), d_y (M x N_out fp32), d_ws / ws_bytes (256-byte aligned,
 * e.g. uw_mlp_stack_workspace_ex with every projection set to UW_PIPE_FULL so that every
 * candidate fits; candidates that do not fit are skipped), decode_stream (or NULL), opts
 * (slots; down_first = the starting order). Out: the layers' pipeline and variant fields,
 * opts.down_first, t_start_ms and t_ms (medians of the starting and the final plan), passes
 * and trials (forwards timed per candidate set). Y and the workspace are overwritten.
 * Errors: UW_EINVAL (arguments, a starting plan that does not fit), any error of the forward.
 */
typedef struct {
    uw_mlp_layer* layers;
    int32_t n_layers;
    int64_t M;
    const uint16_t* d_x;
    float* d_y;
    void* d_ws;
    size_t ws_bytes;
    void* decode_stream;
    uw_stack_opts opts;
    uint32_t pipeline_mask; /* 0 = all five */
    int32_t reps;           /* 0 = 5 */
    int32_t warmup;         /* 0 = 1 */
    int32_t max_passes;     /* 0 = 4 */
    float t_start_ms;
    float t_ms;
    int32_t passes;
    int32_t trials;
} uw_stack_tune_args;

uw_status uw_mlp_stack_autotune(uw_stack_tune_args* args, void* stream);

/*
 * CU-split streams ("Sharing the GPU between decode and compute": the preprocessing of one
 * projection runs on a slice of the compute units while the reconstructive GEMM of another
 * runs on the rest, so neither waits behind the other's workgroups).
 *
 * uw_stream_pair_create (host): two new HIP streams, both at the default priority, on
 * disjoint compute units: decode_cus of the device's CUs (spread evenly over its XCDs) for
 * *decode_stream, all the others for *gemm_stream. Pass them to uw_mlp_stack_forward as
 * (stream, decode_stream), or use them with any entry point; the persistent decoders size
 * their grids to the stream's CUs. The caller owns both and releases them with
 * uw_stream_destroy. Errors: UW_EINVAL (NULL outputs, decode_cus < 1 or >= the device's
 * CUs), UW_EHIP.
 * uw_stream_cu_count (host): the compute units a stream may use (its CU mask; the whole
 * device for the null stream).
 */
uw_status uw_stream_pair_create(int decode_cus, void** gemm_stream, void** decode_stream);
uw_status uw_stream_destroy(void* stream);
uw_status uw_stream_cu_count(void* stream, int* out);

/*
 * uw_stream_read (device). Measurement helper for the HBM roofline ("GPU memory
 * bottleneck": generating a token is bound by the weight bytes read from HBM, not by the
 * arithmetic, so the small-batch GEMM is priced by its bytes): reads d_src[0, bytes)
 * once with a plain streaming kernel on `stream` (eight workgroups per compute unit the
 * stream may use, a grid-stride sweep of 16-byte coalesced loads, sixteen in flight per
 * thread) and computes nothing from it. Timing it with events gives the read rate a kernel that does
 * no other work reaches on this part, the practical ceiling beside the published peak.
 * d_src: device, 16-byte aligned, bytes a multiple of 16 (0 is a no-op); d_sink: one
 * device word the kernel may modify (its value is meaningless). Errors: UW_EINVAL
 * (NULL pointers, misalignment), UW_EHIP.
 */
uw_status uw_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UW_H */
