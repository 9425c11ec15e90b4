// Pipeline execution, the measured autotuner and the SwiGLU glue.
//
// Pipelines ("Four ways to use compressed weights" in the Unweight blog post): full
// decode + plain GEMM, exponent-only decode + reconstructive GEMM, runtime palette
// transcode + reconstructive GEMM, and direct palette (index plane prepared once at
// load). No pipeline wins everywhere ("Why no single pipeline wins"), so the choice per
// matrix and batch size is made by timing every candidate on the target GPU and keeping
// the fastest, which is what the post's autotuner does instead of heuristics.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "uw_internal.h"
#include "uw_recon.h"

namespace uw {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ void fill_kernel(u32x4* p, size_t n16, uint32_t v)
{
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = u32x4{v, v, v, v};
}

// Plain streaming read (the ceiling a kernel that only reads reaches on this part): a
// grid-stride sweep, workgroup b taking the 4 KB pieces b, b + grid, ... so that the whole
// device reads one contiguous region at a time, sixteen pieces in flight per workgroup. Of
// the shapes measured on MI355X (contiguous slices per workgroup, 1 to 16 workgroups per CU,
// 8 or 16 loads in flight) this one reads fastest. The XOR of everything read decides one
// store that the compiler cannot prove dead, so no load is removed.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* src, uint64_t n16, uint32_t* sink)
{
    constexpr int kInFlight = 16;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 256;
    uint32_t acc = 0;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; u++) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kInFlight; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) atomicXor(sink, 1u);
}

// h = bf16(silu(g) * u); eight elements per thread, 16-byte loads and stores.
__global__ void swiglu_kernel(const float* __restrict__ g, const float* __restrict__ u, uint16_t* __restrict__ h,
                              int64_t n)
{
    const int64_t i8 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
    if (i8 + 8 <= n) {
        const floatx4 g0 = *reinterpret_cast<const floatx4*>(g + i8), g1 = *reinterpret_cast<const floatx4*>(g + i8 + 4);
        const floatx4 u0 = *reinterpret_cast<const floatx4*>(u + i8), u1 = *reinterpret_cast<const floatx4*>(u + i8 + 4);
        uint32_t o[8];
        for (int t = 0; t < 4; t++) {
            o[t] = f32_to_bf16_rne(silu_mul(g0[t], u0[t]));
            o[4 + t] = f32_to_bf16_rne(silu_mul(g1[t], u1[t]));
        }
        u32x4 v = {o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)};
        *reinterpret_cast<u32x4*>(h + i8) = v;
    } else {
        for (int64_t i = i8; i < n; i++) h[i] = static_cast<uint16_t>(f32_to_bf16_rne(silu_mul(g[i], u[i])));
    }
}

// Preprocessing slot of uw_run_pipeline_noalloc: a file-scope device array, one per GPU the
// library runs on, held until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from hipGetSymbolAddress, looked
// up once per device (with that device current) and kept in scratch_ptrs.
constexpr size_t kScratchBytes = size_t{128} << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptrs[kMaxDevices] = {};

// Device address of the current device's scratch array (a symbol lookup on the first call
// per device, no allocation).
uw_status scratch_ptr(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(UW_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(UW_EUNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail(UW_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        scratch_ptrs[dev] = p;
    }
    *out = scratch_ptrs[dev];
    return UW_OK;
}

uw_status scrub(void* d, size_t bytes, uint32_t value, hipStream_t s)
{
    const size_t n16 = bytes / 16;
    if (!n16) return UW_OK;
    hipLaunchKernelGGL(fill_kernel, dim3(2048), dim3(256), 0, s, static_cast<u32x4*>(d), n16, value);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? UW_OK : fail(UW_EHIP, "scrub launch failed: %s", hipGetErrorString(e));
}

}  // namespace

}  // namespace uw

using namespace uw;

extern "C" {

uw_status uw_run_pipeline(int32_t pipeline, int32_t variant, int32_t split_k, const uw_header* h, const void* d_blob,
                          const uint8_t* d_direct, int64_t M, const uint16_t* d_x, int64_t ldx, float* d_y, int64_t ldy,
                          void* d_ws, size_t ws_bytes, uint32_t* d_err, void* stream)
{
    clear_error();
    if (!h) return fail(UW_EINVAL, "NULL header");
    size_t need = 0;
    uw_status st = uw_workspace_bytes(h, pipeline, &need);
    if (st != UW_OK) return st;
    if (need > 0 && (!d_ws || ws_bytes < need)) return fail(UW_ENOSPACE, "pipeline %d needs %zu workspace bytes", pipeline, need);
    uw_gemm_args g;
    std::memset(&g, 0, sizeof g);
    g.M = M;
    g.d_x = d_x;
    g.ldx = ldx;
    g.h = h;
    g.d_blob = d_blob;
    g.d_y = d_y;
    g.ldy = ldy;
    g.variant = variant;
    g.split_k = split_k;
    switch (pipeline) {
    case UW_PIPE_FULL:
        if ((st = uw_decode_full(h, d_blob, static_cast<uint16_t*>(d_ws), d_err, stream)) != UW_OK) return st;
        g.src = UW_W_BF16;
        g.d_wplane = d_ws;
        break;
    case UW_PIPE_EXP:
        if ((st = uw_decode_exponent(h, d_blob, static_cast<uint8_t*>(d_ws), d_err, stream)) != UW_OK) return st;
        g.src = UW_W_EXP;
        g.d_wplane = d_ws;
        break;
    case UW_PIPE_TRANSCODE:
        if ((st = uw_transcode_palette(h, d_blob, static_cast<uint8_t*>(d_ws), d_err, stream)) != UW_OK) return st;
        g.src = UW_W_IDX;
        g.d_wplane = d_ws;
        break;
    case UW_PIPE_DIRECT:
        if (!d_direct) return fail(UW_EINVAL, "direct palette needs the direct plane (uw_prepare_direct)");
        g.src = UW_W_DIRECT;
        g.d_wplane = d_direct;
        break;
    case UW_PIPE_EXPAND:
        if (!d_direct) return fail(UW_EINVAL, "the expand pipeline needs the direct plane (uw_prepare_direct)");
        if ((st = uw_expand_direct(h, d_direct, static_cast<uint16_t*>(d_ws), stream)) != UW_OK) return st;
        g.src = UW_W_BF16;
        g.d_wplane = d_ws;
        break;
    default: return fail(UW_EINVAL, "unknown pipeline %d", pipeline);
    }
    return uw_recon_gemm(&g, stream);
}

uw_status uw_run_pipeline_noalloc(int32_t pipeline, int32_t variant, int32_t split_k, const uw_header* h,
                                  const void* d_blob, const uint8_t* d_direct, int64_t M, const uint16_t* d_x,
                                  int64_t ldx, float* d_y, int64_t ldy, uint32_t* d_err, void* stream)
{
    clear_error();
    if (!h) return fail(UW_EINVAL, "NULL header");
    size_t need = 0;
    uw_status st = uw_workspace_bytes(h, pipeline, &need);
    if (st != UW_OK) return st;
    if (need > kScratchBytes)
        return fail(UW_ENOSPACE, "pipeline %d needs %zu bytes of preprocessing slot; the allocation-free entry point has %zu",
                    pipeline, need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0 && (st = scratch_ptr(&ws)) != UW_OK) return st;
    // the decoders overwrite every byte of the plane they write, so nothing is cleared
    return uw_run_pipeline(pipeline, variant, split_k, h, d_blob, d_direct, M, d_x, ldx, d_y, ldy, ws, need, d_err,
                           stream);
}

size_t uw_noalloc_scratch_bytes(void) { return kScratchBytes; }

uw_status uw_autotune(const uw_tune_args* a, const int64_t* Ms, int nM, void* stream, uw_plan* out)
{
    try {
        clear_error();
        if (!a || !a->h || !Ms || !out || nM < 0) return fail(UW_EINVAL, "NULL argument");
        const uw_header* h = a->h;
        const int reps = a->reps > 0 ? a->reps : 10;
        const int warmup = a->warmup > 0 ? a->warmup : 2;
        const int trials = a->trials > 0 ? a->trials : 3;
        const uint32_t pmask = a->pipeline_mask ? a->pipeline_mask : 0x1Fu;
        const uint32_t vmask = a->variant_mask ? static_cast<uint32_t>(a->variant_mask) : 0xFFFFFFFFu;
        // the rotation set: the caller's matrices of this shape, or the single one
        std::vector<uw_proj> rot;
        if (a->rot && a->n_rot > 0) {
            rot.assign(a->rot, a->rot + a->n_rot);
        } else {
            uw_proj one;
            std::memset(&one, 0, sizeof one);
            one.h = h;
            one.d_blob = a->d_blob;
            one.d_direct = a->d_direct;
            rot.push_back(one);
        }
        bool all_direct = true;
        for (const uw_proj& r : rot) {
            if (!r.h || !r.d_blob) return fail(UW_EINVAL, "rotation entry with a NULL header or blob");
            if (r.h->N != h->N || r.h->K != h->K) return fail(UW_EINVAL, "rotation entries must have the header's N and K");
            all_direct = all_direct && r.d_direct;
        }
        for (int mi = 0; mi < nM; mi++)
            if (Ms[mi] < 1) return fail(UW_ESHAPE, "M must be >= 1");
        hipStream_t s = static_cast<hipStream_t>(stream);
        hipEvent_t e0, e1;
        if (hipEventCreate(&e0) != hipSuccess) return fail(UW_EHIP, "hipEventCreate failed");
        if (hipEventCreate(&e1) != hipSuccess) {
            (void)hipEventDestroy(e0);
            return fail(UW_EHIP, "hipEventCreate failed");
        }
        const uint32_t G = static_cast<uint32_t>(h->K / 64);
        uw_status result = UW_OK;
        size_t next = 0;  // position in the rotation, carried across candidates
        for (int mi = 0; mi < nM && result == UW_OK; mi++) {
            const int64_t M = Ms[mi];
            // one forward of candidate (p, v, ks) on the next matrix of the rotation
            auto run = [&](int p, int v, int ks) -> uw_status {
                const uw_proj& r = rot[next];
                next = (next + 1) % rot.size();
                return uw_run_pipeline(p, v, ks, r.h, r.d_blob, r.d_direct, M, a->d_x, h->K, a->d_y, h->N, a->d_ws,
                                       a->ws_bytes, nullptr, stream);
            };
            uw_plan best;
            best.pipeline = -1;
            best.variant = -1;
            best.t_ms = 3.0e38f;
            best.split_k = 0;
            for (int p = 0; p < kPipelines && result == UW_OK; p++) {
                if (!(pmask >> p & 1u)) continue;
                if ((p == UW_PIPE_DIRECT || p == UW_PIPE_EXPAND) && !all_direct) continue;
                size_t need = 0;
                uw_workspace_bytes(h, p, &need);
                if (need > a->ws_bytes || (need > 0 && !a->d_ws)) continue;
                const int32_t src = p == UW_PIPE_FULL || p == UW_PIPE_EXPAND ? UW_W_BF16 : p == UW_PIPE_EXP ? UW_W_EXP
                                    : p == UW_PIPE_TRANSCODE ? UW_W_IDX : UW_W_DIRECT;
                for (int v = 0; v < uw_variant_count() && result == UW_OK; v++) {
                    if (!(vmask >> v & 1u) || !uw_variant_supports(v, h->N, h->K, M, src)) continue;
                    // the variant's own split, then (tune_split) the listed counts it does not
                    // already cover; each count as the launch will round it
                    std::vector<int> splits = {uw_split_count(v, h->N, h->K, M, 0)};
                    if (a->tune_split) {
                        for (int want : {1, 2, 3, 4, 6, 8}) {
                            if (static_cast<uint32_t>(want) > G / 8 && want > 1) continue;
                            const int got = uw_split_count(v, h->N, h->K, M, want);
                            if (got > 0 && std::find(splits.begin(), splits.end(), got) == splits.end()) splits.push_back(got);
                        }
                    }
                    for (int ks : splits) {
                        std::vector<float> t;
                        for (int r = 0; r < warmup && result == UW_OK; r++) {
                            uw_status st = run(p, v, ks);
                            if (st == UW_EUNSUPPORTED) {  // a variant this problem cannot use: not a candidate
                                clear_error();
                                result = UW_EUNSUPPORTED;
                            } else if (st != UW_OK) {
                                result = st;
                            }
                        }
                        if (result == UW_EUNSUPPORTED) {
                            result = UW_OK;
                            continue;
                        }
                        for (int tr = 0; tr < trials && result == UW_OK; tr++) {
                            if (a->d_scrub && (result = scrub(a->d_scrub, a->scrub_bytes, static_cast<uint32_t>(tr), s)) != UW_OK)
                                break;
                            if (hipEventRecord(e0, s) != hipSuccess) { result = fail(UW_EHIP, "event record failed"); break; }
                            for (int r = 0; r < reps && result == UW_OK; r++) result = run(p, v, ks);
                            if (result != UW_OK) break;
                            if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) {
                                result = fail(UW_EHIP, "event synchronize failed");
                                break;
                            }
                            float ms = 0.f;
                            (void)hipEventElapsedTime(&ms, e0, e1);
                            t.push_back(ms / static_cast<float>(reps));
                        }
                        if (result != UW_OK || t.empty()) break;
                        std::sort(t.begin(), t.end());
                        const float med = t[t.size() / 2];
                        if (med < best.t_ms) {
                            best.pipeline = p;
                            best.variant = v;
                            best.t_ms = med;
                            best.split_k = ks;
                        }
                    }
                }
            }
            if (result == UW_OK && best.pipeline < 0) result = fail(UW_EUNSUPPORTED, "no candidate fits M=%lld", (long long)M);
            out[mi] = best;
        }
        (void)hipEventDestroy(e0);
        (void)hipEventDestroy(e1);
        return result;
    } catch (...) {
        return fail(UW_EINTERNAL, "unexpected exception in uw_autotune");
    }
}

uw_status uw_swiglu(const float* d_g, const float* d_u, int64_t n, uint16_t* d_h, void* stream)
{
    clear_error();
    if (n < 0) return fail(UW_ESHAPE, "n < 0");
    if (n == 0) return UW_OK;
    if (!d_g || !d_u || !d_h) return fail(UW_EINVAL, "NULL device pointer");
    if (!aligned(d_g, 16) || !aligned(d_u, 16) || !aligned(d_h, 16)) return fail(UW_EINVAL, "pointers must be 16-byte aligned");
    const int64_t threads = (n + 7) / 8;
    const dim3 grid(static_cast<uint32_t>((threads + 255) / 256));
    hipLaunchKernelGGL(swiglu_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), d_g, d_u, d_h, n);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? UW_OK : fail(UW_EHIP, "swiglu launch failed: %s", hipGetErrorString(e));
}

namespace {

struct StackLayout {
    int64_t Nff, K, Nout;
    size_t g, u, h, slot0, slot_bytes, total;
    int slots;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

const uw_proj& role_of(const uw_mlp_layer& L, int r) { return r == 0 ? L.gate : r == 1 ? L.up : L.down; }

// Workspace of a stack forward: g, u (fp32 M x N_ff), h (bf16 M x N_ff), then `slots` decode
// slots of the largest plane any projection's pipeline decodes.
uw_status stack_layout(const uw_mlp_layer* L, int n, int64_t M, int slots, StackLayout* o)
{
    if (!L || n <= 0) return fail(UW_EINVAL, "no layers");
    if (M < 0) return fail(UW_ESHAPE, "M < 0");
    if (slots < 1 || slots > 8) return fail(UW_EINVAL, "decode slots must be 1..8, not %d", slots);
    const uw_header* g0 = L[0].gate.h;
    const uw_header* d0 = L[0].down.h;
    if (!g0 || !d0) return fail(UW_EINVAL, "NULL header");
    o->Nff = g0->N;
    o->K = g0->K;
    o->Nout = d0->N;
    size_t slot = 0;
    for (int l = 0; l < n; l++) {
        for (int q = 0; q < 3; q++) {
            const uw_proj& pr = role_of(L[l], q);
            if (!pr.h || !pr.d_blob) return fail(UW_EINVAL, "layer %d projection %d: NULL header or blob", l, q);
            if ((pr.pipeline == UW_PIPE_DIRECT || pr.pipeline == UW_PIPE_EXPAND) && !pr.d_direct)
                return fail(UW_EINVAL, "layer %d projection %d: pipeline %d needs the direct plane", l, q, pr.pipeline);
            size_t need = 0;
            uw_status st = uw_workspace_bytes(pr.h, pr.pipeline, &need);
            if (st != UW_OK) return st;
            slot = need > slot ? need : slot;
        }
        const uw_header* g = L[l].gate.h;
        const uw_header* u = L[l].up.h;
        const uw_header* d = L[l].down.h;
        if (g->N != o->Nff || g->K != o->K || u->N != o->Nff || u->K != o->K || d->K != o->Nff || d->N != o->Nout)
            return fail(UW_ESHAPE, "layer %d: shapes differ from layer 0 or do not chain", l);
    }
    const size_t mf = static_cast<size_t>(M) * static_cast<size_t>(o->Nff);
    o->slots = slots;
    o->slot_bytes = align256(slot);
    o->g = 0;
    o->u = align256(4 * mf);
    o->h = o->u + align256(4 * mf);
    o->slot0 = o->h + align256(2 * mf);
    o->total = o->slot0 + static_cast<size_t>(slots) * o->slot_bytes;
    return UW_OK;
}

// Decode one projection's plane into `slot` (no-op for direct palette).
uw_status decode_proj(const uw_proj& p, void* slot, void* stream)
{
    switch (p.pipeline) {
    case UW_PIPE_FULL: return uw_decode_full(p.h, p.d_blob, static_cast<uint16_t*>(slot), nullptr, stream);
    case UW_PIPE_EXP: return uw_decode_exponent(p.h, p.d_blob, static_cast<uint8_t*>(slot), nullptr, stream);
    case UW_PIPE_TRANSCODE: return uw_transcode_palette(p.h, p.d_blob, static_cast<uint8_t*>(slot), nullptr, stream);
    case UW_PIPE_DIRECT: return UW_OK;
    case UW_PIPE_EXPAND: return uw_expand_direct(p.h, p.d_direct, static_cast<uint16_t*>(slot), stream);
    default: return fail(UW_EINVAL, "unknown pipeline %d", p.pipeline);
    }
}

// GEMM arguments of a projection whose plane is ready (in `slot`, or the direct plane).
uw_gemm_args proj_args(const uw_proj& p, const void* slot, int64_t M, const uint16_t* x, int64_t ldx, float* y,
                       int64_t ldy)
{
    uw_gemm_args g;
    std::memset(&g, 0, sizeof g);
    g.M = M;
    g.d_x = x;
    g.ldx = ldx;
    g.h = p.h;
    g.d_blob = p.d_blob;
    g.d_y = y;
    g.ldy = ldy;
    g.variant = p.variant;
    g.split_k = p.split_k;
    g.src = p.pipeline == UW_PIPE_FULL || p.pipeline == UW_PIPE_EXPAND ? UW_W_BF16 : p.pipeline == UW_PIPE_EXP ? UW_W_EXP
          : p.pipeline == UW_PIPE_TRANSCODE ? UW_W_IDX : UW_W_DIRECT;
    g.d_wplane = p.pipeline == UW_PIPE_DIRECT ? static_cast<const void*>(p.d_direct) : slot;
    return g;
}

// The GEMM of a projection whose plane is ready.
uw_status gemm_proj(const uw_proj& p, const void* slot, int64_t M, const uint16_t* x, int64_t ldx, float* y, int64_t ldy,
                    void* stream, bool y_zeroed = false)
{
    const uw_gemm_args g = proj_args(p, slot, M, x, ldx, y, ldy);
    return launch_gemm(&g, stream, y_zeroed);
}

// The up projection's GEMM with the SwiGLU in its epilogue (h = bf16(silu(g) u), g the gate's
// output, u never stored); where the variant or a K split leaves no such epilogue, the GEMM
// into u and the separate activation kernel.
uw_status up_proj_swiglu(const uw_proj& p, const void* slot, int64_t M, const uint16_t* x, int64_t ldx, const float* g,
                         float* u, uint16_t* h, int64_t ldf, void* stream)
{
    const uw_gemm_args a = proj_args(p, slot, M, x, ldx, const_cast<float*>(g), ldf);  // Y = g, read only
    uw_status st = launch_gemm_swiglu(&a, h, ldf, stream);
    if (st != UW_EUNSUPPORTED) return st;
    clear_error();
    if ((st = gemm_proj(p, slot, M, x, ldx, u, ldf, stream)) != UW_OK) return st;
    return uw_swiglu(g, u, M * p.h->N, h, stream);
}

// gate, up and SwiGLU of a layer in one launch when both projections are direct planes
// and the fused form applies; UW_EUNSUPPORTED otherwise (the caller runs them one by one).
uw_status gate_up_fused(const uw_proj& gp, const uw_proj& up, int64_t M, const uint16_t* x, int64_t ldx, float* g,
                        float* u, uint16_t* h, int64_t ldf, void* stream, const ZeroTarget* clear = nullptr)
{
    if (gp.pipeline != UW_PIPE_DIRECT || up.pipeline != UW_PIPE_DIRECT || M > 64) return UW_EUNSUPPORTED;
    uw_gemm_args a[2];
    const uw_proj* pr[2] = {&gp, &up};
    float* y[2] = {g, u};
    for (int q = 0; q < 2; q++) {
        std::memset(&a[q], 0, sizeof a[q]);
        a[q].M = M;
        a[q].d_x = x;
        a[q].ldx = ldx;
        a[q].h = pr[q]->h;
        a[q].d_blob = pr[q]->d_blob;
        a[q].src = UW_W_DIRECT;
        a[q].d_wplane = pr[q]->d_direct;
        a[q].d_y = y[q];
        a[q].ldy = ldf;
        a[q].variant = pr[q]->variant;
        a[q].split_k = pr[q]->split_k;
    }
    return launch_gate_up_gemm(&a[0], &a[1], h, ldf, stream, clear);
}

// ---- the schedule of a forward with a decode stream
//
// A layer whose projections all read direct planes needs no preprocessing (an "easy"
// layer); any other is "hard" ("Sharing the GPU between decode and compute": the
// preprocessing of the next hard layer runs on a side stream while easy layers compute,
// through double-buffered slots; down is consumed last in a layer, so its decode can be
// issued first). Every decode-first projection gets a decode index q in decode order (per
// layer gate, up, down, or down first) and slot q mod S. The plan is built on the host
// before anything is launched: after each GEMM that frees a slot, every decode whose slot
// is free is issued at once, so decodes run as far ahead of their GEMMs as the slots
// allow. A decode order that would need a slot still held by a later GEMM is rejected.
struct Action {
    enum Kind { DECODE, GEMM, FUSED, SWIGLU } kind;
    int layer, role, q;  // role 0 gate, 1 up, 2 down; q = decode index or -1
};

bool both_direct(const uw_mlp_layer& L, int64_t M)
{
    return L.gate.pipeline == UW_PIPE_DIRECT && L.up.pipeline == UW_PIPE_DIRECT && M <= 64;
}

uw_status build_plan(const uw_mlp_layer* layers, int n, int64_t M, int S, bool down_first, std::vector<Action>& plan)
{
    plan.clear();
    std::vector<std::pair<int, int>> dec;
    std::vector<int> qof(static_cast<size_t>(3) * n, -1);
    static const int kInOrder[3] = {0, 1, 2}, kDownFirst[3] = {2, 0, 1};
    for (int l = 0; l < n; l++) {
        const int* order = down_first ? kDownFirst : kInOrder;
        for (int k = 0; k < 3; k++) {
            const int r = order[k];
            if (role_of(layers[l], r).pipeline == UW_PIPE_DIRECT) continue;
            qof[3 * l + r] = static_cast<int>(dec.size());
            dec.push_back({l, r});
        }
    }
    std::vector<char> consumed(dec.size(), 0);
    size_t next = 0;
    auto pump = [&]() {
        while (next < dec.size() && (next < static_cast<size_t>(S) || consumed[next - S])) {
            plan.push_back({Action::DECODE, dec[next].first, dec[next].second, static_cast<int>(next)});
            next++;
        }
    };
    pump();
    for (int l = 0; l < n; l++) {
        auto gemm = [&](int r) -> bool {
            const int q = qof[3 * l + r];
            if (q >= 0 && static_cast<size_t>(q) >= next) return false;
            plan.push_back({Action::GEMM, l, r, q});
            if (q >= 0) {
                consumed[q] = 1;
                pump();
            }
            return true;
        };
        if (both_direct(layers[l], M)) {
            plan.push_back({Action::FUSED, l, -1, -1});
        } else {
            if (!gemm(0) || !gemm(1))
                return fail(UW_EINVAL, "layer %d: this decode order needs more than %d decode slots", l, S);
            plan.push_back({Action::SWIGLU, l, -1, -1});
        }
        if (!gemm(2)) return fail(UW_EINVAL, "layer %d: this decode order needs more than %d decode slots", l, S);
    }
    return UW_OK;
}

uw_status stack_forward(const uw_mlp_layer* layers, int n_layers, int64_t M, const uint16_t* d_x, float* d_y, void* d_ws,
                        size_t ws_bytes, void* stream, void* decode_stream, int slots, bool down_first)
{
    StackLayout lay;
    uw_status st = stack_layout(layers, n_layers, M, slots, &lay);
    if (st != UW_OK) return st;
    if (M == 0) return UW_OK;
    if (!d_x || !d_y || !d_ws) return fail(UW_EINVAL, "NULL device pointer");
    if (!aligned(d_ws, 256)) return fail(UW_EINVAL, "d_ws must be 256-byte aligned");
    if (ws_bytes < lay.total) return fail(UW_ENOSPACE, "the stack needs %zu workspace bytes", lay.total);
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    float* g = reinterpret_cast<float*>(ws + lay.g);
    float* u = reinterpret_cast<float*>(ws + lay.u);
    uint16_t* h = reinterpret_cast<uint16_t*>(ws + lay.h);
    auto slot = [&](int s) -> void* { return ws + lay.slot0 + static_cast<size_t>(s) * lay.slot_bytes; };
    const int64_t mf = M * lay.Nff;
    // operands of a projection's GEMM
    auto gemm_io = [&](int r, const uint16_t*& x, int64_t& ldx, float*& y, int64_t& ldy) {
        if (r == 2) {
            x = h;
            ldx = lay.Nff;
            y = d_y;
            ldy = lay.Nout;
        } else {
            x = d_x;
            ldx = lay.K;
            y = r == 0 ? g : u;
            ldy = lay.Nff;
        }
    };
    // gate, up and SwiGLU of a layer whose gate and up are direct planes; with `clear`, the
    // fused launch also clears that Y (*cleared tells whether it ran)
    auto direct_pair = [&](const uw_mlp_layer& L, void* s, const ZeroTarget* clear = nullptr,
                           bool* cleared = nullptr) -> uw_status {
        uw_status r = gate_up_fused(L.gate, L.up, M, d_x, lay.K, g, u, h, lay.Nff, s, clear);
        if (cleared) *cleared = r == UW_OK && clear;
        if (r != UW_EUNSUPPORTED) return r;
        clear_error();
        if ((r = gemm_proj(L.gate, nullptr, M, d_x, lay.K, g, lay.Nff, s)) != UW_OK) return r;
        return up_proj_swiglu(L.up, nullptr, M, d_x, lay.K, g, u, h, lay.Nff, s);
    };

    if (!decode_stream) {
        for (int l = 0; l < n_layers && st == UW_OK; l++) {
            const uw_mlp_layer& L = layers[l];
            // a K-split down adds into Y: the fused gate/up launch before it clears Y, which
            // saves the split launch a clearing launch of its own
            const bool split_down =
                lay.Nout % 4 == 0 && uw_split_count(L.down.variant, lay.Nout, lay.Nff, M, L.down.split_k) > 1;
            const ZeroTarget clear_y = {d_y, lay.Nout, M, lay.Nout};
            bool cleared = false;
            if (both_direct(L, M)) {
                st = direct_pair(L, stream, split_down ? &clear_y : nullptr, &cleared);
            } else {
                if ((st = decode_proj(L.gate, slot(0), stream)) == UW_OK)
                    st = gemm_proj(L.gate, slot(0), M, d_x, lay.K, g, lay.Nff, stream);
                if (st == UW_OK && (st = decode_proj(L.up, slot(0), stream)) == UW_OK)
                    st = up_proj_swiglu(L.up, slot(0), M, d_x, lay.K, g, u, h, lay.Nff, stream);
            }
            if (st != UW_OK) break;
            if ((st = decode_proj(L.down, slot(0), stream)) != UW_OK) break;
            st = gemm_proj(L.down, slot(0), M, h, lay.Nff, d_y, lay.Nout, stream, cleared);
        }
        return st;
    }

    std::vector<Action> plan;
    if ((st = build_plan(layers, n_layers, M, slots, down_first, plan)) != UW_OK) return st;
    hipStream_t ms = static_cast<hipStream_t>(stream), ds = static_cast<hipStream_t>(decode_stream);
    std::vector<hipEvent_t> decoded(slots, nullptr), freed(slots, nullptr);
    hipEvent_t start = nullptr;
    auto release = [&]() {
        for (int s = 0; s < slots; s++) {
            if (decoded[s]) (void)hipEventDestroy(decoded[s]);
            if (freed[s]) (void)hipEventDestroy(freed[s]);
        }
        if (start) (void)hipEventDestroy(start);
    };
    for (int s = 0; s < slots; s++) {
        if (hipEventCreateWithFlags(&decoded[s], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&freed[s], hipEventDisableTiming) != hipSuccess) {
            release();
            return fail(UW_EHIP, "hipEventCreate failed");
        }
    }
    // the decode stream must also see everything queued on the main stream so far (the
    // caller's writes of X and of the planes)
    if (hipEventCreateWithFlags(&start, hipEventDisableTiming) != hipSuccess || hipEventRecord(start, ms) != hipSuccess ||
        hipStreamWaitEvent(ds, start, 0) != hipSuccess) {
        release();
        return fail(UW_EHIP, "stream ordering failed");
    }
    std::vector<char> swiglu_done(n_layers, 0);  // the layer's up GEMM ran the SwiGLU in its epilogue
    for (const Action& a : plan) {
        const uw_mlp_layer& L = layers[a.layer];
        if (a.kind == Action::DECODE) {
            const int s = a.q % slots;
            if (a.q >= slots && hipStreamWaitEvent(ds, freed[s], 0) != hipSuccess) { st = fail(UW_EHIP, "wait failed"); break; }
            if ((st = decode_proj(role_of(L, a.role), slot(s), ds)) != UW_OK) break;
            if (hipEventRecord(decoded[s], ds) != hipSuccess) { st = fail(UW_EHIP, "event record failed"); break; }
        } else if (a.kind == Action::GEMM) {
            const uint16_t* x;
            int64_t ldx, ldy;
            float* y;
            gemm_io(a.role, x, ldx, y, ldy);
            auto run = [&](const void* sl) -> uw_status {
                if (a.role != 1) return gemm_proj(role_of(L, a.role), sl, M, x, ldx, y, ldy, ms);
                swiglu_done[a.layer] = 1;  // h is written either way: by the epilogue or the activation kernel
                return up_proj_swiglu(L.up, sl, M, d_x, lay.K, g, u, h, lay.Nff, ms);
            };
            if (a.q < 0) {
                if ((st = run(nullptr)) != UW_OK) break;
                continue;
            }
            const int s = a.q % slots;
            if (hipStreamWaitEvent(ms, decoded[s], 0) != hipSuccess) { st = fail(UW_EHIP, "wait failed"); break; }
            if ((st = run(slot(s))) != UW_OK) break;
            if (hipEventRecord(freed[s], ms) != hipSuccess) { st = fail(UW_EHIP, "event record failed"); break; }
        } else if (a.kind == Action::FUSED) {
            if ((st = direct_pair(L, ms)) != UW_OK) break;
        } else if (!swiglu_done[a.layer]) {
            if ((st = uw_swiglu(g, u, mf, h, ms)) != UW_OK) break;
        }
    }
    release();
    return st;
}

int opt_slots(const uw_stack_opts* o) { return o && o->slots != 0 ? o->slots : 2; }  // 0 = 2; out of range: EINVAL

}  // namespace

uw_status uw_mlp_stack_workspace(const uw_mlp_layer* layers, int n_layers, int64_t M, int two_slots, size_t* out)
{
    clear_error();
    if (!out) return fail(UW_EINVAL, "NULL argument");
    StackLayout lay;
    uw_status st = stack_layout(layers, n_layers, M, two_slots ? 2 : 1, &lay);
    if (st == UW_OK) *out = lay.total;
    return st;
}

uw_status uw_mlp_stack_workspace_ex(const uw_mlp_layer* layers, int n_layers, int64_t M, const uw_stack_opts* opts,
                                    size_t* out)
{
    clear_error();
    if (!out) return fail(UW_EINVAL, "NULL argument");
    StackLayout lay;
    uw_status st = stack_layout(layers, n_layers, M, opt_slots(opts), &lay);
    if (st == UW_OK) *out = lay.total;
    return st;
}

uw_status uw_mlp_stack_forward(const uw_mlp_layer* layers, int n_layers, int64_t M, const uint16_t* d_x, float* d_y,
                               void* d_ws, size_t ws_bytes, void* stream, void* decode_stream)
{
    try {
        clear_error();
        return stack_forward(layers, n_layers, M, d_x, d_y, d_ws, ws_bytes, stream, decode_stream, decode_stream ? 2 : 1,
                             false);
    } catch (...) {
        return fail(UW_EINTERNAL, "unexpected exception in uw_mlp_stack_forward");
    }
}

uw_status uw_mlp_stack_forward_ex(const uw_mlp_layer* layers, int n_layers, int64_t M, const uint16_t* d_x, float* d_y,
                                  void* d_ws, size_t ws_bytes, void* stream, void* decode_stream, const uw_stack_opts* opts)
{
    try {
        clear_error();
        return stack_forward(layers, n_layers, M, d_x, d_y, d_ws, ws_bytes, stream, decode_stream, opt_slots(opts),
                             opts && opts->down_first);
    } catch (...) {
        return fail(UW_EINTERNAL, "unexpected exception in uw_mlp_stack_forward_ex");
    }
}

// ---- coordinate-descent tuning of a whole stack ("Why no single pipeline wins" and
// "Sharing the GPU between decode and compute": the runtime's per-projection choices are
// measured end to end, one coordinate at a time, until a pass changes nothing)
uw_status uw_mlp_stack_autotune(uw_stack_tune_args* a, void* stream)
{
    try {
        clear_error();
        if (!a || !a->layers || a->n_layers <= 0) return fail(UW_EINVAL, "NULL argument or no layers");
        const int n = a->n_layers;
        uw_mlp_layer* L = a->layers;
        const int reps = a->reps > 0 ? a->reps : 5, warmup = a->warmup > 0 ? a->warmup : 1;
        const int max_passes = a->max_passes > 0 ? a->max_passes : 4;
        const uint32_t pmask = a->pipeline_mask ? a->pipeline_mask : 0x1Fu;
        const int slots = opt_slots(&a->opts);
        // layer class: 0 when all three projections have direct planes ("easy" once they
        // use them), 1 otherwise (a "hard" layer, which always needs preprocessing)
        std::vector<int> cls(n);
        bool present[2] = {false, false};
        for (int l = 0; l < n; l++) {
            cls[l] = L[l].gate.d_direct && L[l].up.d_direct && L[l].down.d_direct ? 0 : 1;
            present[cls[l]] = true;
        }
        uw_stack_opts opts = a->opts;
        opts.slots = slots;
        auto fits = [&]() -> bool {
            StackLayout lay;
            if (stack_layout(L, n, a->M, a->decode_stream ? slots : 1, &lay) != UW_OK) {
                clear_error();
                return false;
            }
            if (lay.total > a->ws_bytes) return false;
            if (!a->decode_stream) return true;
            std::vector<Action> plan;
            if (build_plan(L, n, a->M, slots, opts.down_first != 0, plan) != UW_OK) {
                clear_error();
                return false;
            }
            return true;
        };
        if (!fits()) return fail(UW_EINVAL, "the starting plan does not run in this workspace / slot count");
        hipStream_t s = static_cast<hipStream_t>(stream);
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
            if (e0) (void)hipEventDestroy(e0);
            return fail(UW_EHIP, "hipEventCreate failed");
        }
        int trials = 0;
        auto measure = [&](float& med) -> uw_status {
            std::vector<float> t;
            for (int r = 0; r < warmup + reps; r++) {
                if (r >= warmup && hipEventRecord(e0, s) != hipSuccess) return fail(UW_EHIP, "event record failed");
                uw_status st = stack_forward(L, n, a->M, a->d_x, a->d_y, a->d_ws, a->ws_bytes, stream, a->decode_stream,
                                             a->decode_stream ? slots : 1, opts.down_first != 0);
                if (st != UW_OK) return st;
                if (r >= warmup) {
                    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)
                        return fail(UW_EHIP, "event synchronize failed");
                    float ms = 0.f;
                    (void)hipEventElapsedTime(&ms, e0, e1);
                    t.push_back(ms);
                }
            }
            std::sort(t.begin(), t.end());
            med = t[t.size() / 2];
            trials++;
            return UW_OK;
        };
        // coordinate (class, role): set every layer of the class to pipeline p (default
        // variant and K split)
        auto get = [&](int c, int r) -> int {
            for (int l = 0; l < n; l++)
                if (cls[l] == c) return role_of(L[l], r).pipeline;
            return -1;
        };
        std::vector<uw_mlp_layer> saved(L, L + n);
        auto set = [&](int c, int r, int p) {
            for (int l = 0; l < n; l++) {
                if (cls[l] != c) continue;
                uw_proj& pr = r == 0 ? L[l].gate : r == 1 ? L[l].up : L[l].down;
                pr.pipeline = p;
                pr.variant = -1;
                pr.split_k = 0;
            }
        };
        float best = 0.f;
        uw_status st = measure(best);
        a->t_start_ms = best;
        int pass = 0;
        for (; st == UW_OK && pass < max_passes; pass++) {
            bool changed = false;
            for (int c = 0; c < 2 && st == UW_OK; c++) {
                if (!present[c]) continue;
                for (int r = 0; r < 3 && st == UW_OK; r++) {
                    for (int p = 0; p < kPipelines && st == UW_OK; p++) {
                        const int cur = get(c, r);
                        if (p == cur || !(pmask >> p & 1u)) continue;
                        if ((p == UW_PIPE_DIRECT || p == UW_PIPE_EXPAND) && c == 1) {
                            // a hard layer may still hold a direct plane for this projection
                            bool all = true;
                            for (int l = 0; l < n; l++)
                                if (cls[l] == 1 && !role_of(L[l], r).d_direct) all = false;
                            if (!all) continue;
                        }
                        saved.assign(L, L + n);
                        set(c, r, p);
                        float t = 0.f;
                        if (fits() && (st = measure(t)) == UW_OK && t < best * 0.99f) {
                            best = t;
                            changed = true;
                        } else {
                            std::copy(saved.begin(), saved.end(), L);
                        }
                    }
                }
            }
            // the decode order, where a decode stream with room for a whole layer is given
            if (st == UW_OK && a->decode_stream && slots >= 3) {
                opts.down_first = !opts.down_first;
                float t = 0.f;
                if (fits() && (st = measure(t)) == UW_OK && t < best * 0.99f) {
                    best = t;
                    changed = true;
                } else {
                    opts.down_first = !opts.down_first;
                }
            }
            if (!changed) {
                pass++;
                break;
            }
        }
        (void)hipEventDestroy(e0);
        (void)hipEventDestroy(e1);
        a->opts.down_first = opts.down_first;
        a->t_ms = best;
        a->passes = pass;
        a->trials = trials;
        return st;
    } catch (...) {
        return fail(UW_EINTERNAL, "unexpected exception in uw_mlp_stack_autotune");
    }
}

// ---------------------------------------------------------------- CU-split streams
// Decode next to the GEMM ("Sharing the GPU between decode and compute"): two streams on
// disjoint compute units, so a projection's preprocessing can run beside another's
// reconstructive GEMM without either queueing behind the other's workgroups.
uw_status uw_stream_pair_create(int decode_cus, void** gemm_stream, void** decode_stream)
{
    using namespace uw;
    clear_error();
    if (!gemm_stream || !decode_stream) return fail(UW_EINVAL, "NULL output");
    if (decode_cus < 1) return fail(UW_EINVAL, "decode_cus must be >= 1");
    const uint32_t T = cu_count();
    if (static_cast<uint32_t>(decode_cus) >= T) return fail(UW_EINVAL, "decode_cus must be < %u", T);
    // The decoder's compute units are spread over the XCDs (T / 8 CUs each when T % 8 == 0):
    // XCD x gives its share at positions k * P / n + x (mod P), so whether the mask bits
    // number the CUs XCD by XCD or round-robin over the XCDs, every XCD keeps both kinds.
    const uint32_t X = T % 8 == 0 ? 8 : 1, P = T / X, d = static_cast<uint32_t>(decode_cus);
    const uint32_t words = (T + 31) / 32;
    std::vector<uint32_t> dm(words, 0u), gm(words, 0u);
    for (uint32_t i = 0; i < T; i++) gm[i / 32] |= 1u << (i % 32);
    for (uint32_t x = 0; x < X; x++) {
        const uint32_t n = d / X + (x < d % X ? 1u : 0u);
        for (uint32_t k = 0; k < n; k++) {
            const uint32_t i = x * P + (k * P / n + x) % P;
            dm[i / 32] |= 1u << (i % 32);
            gm[i / 32] &= ~(1u << (i % 32));
        }
    }
    hipStream_t g = nullptr, dd = nullptr;
    if (hipExtStreamCreateWithCUMask(&g, words, gm.data()) != hipSuccess)
        return fail(UW_EHIP, "hipExtStreamCreateWithCUMask failed");
    if (hipExtStreamCreateWithCUMask(&dd, words, dm.data()) != hipSuccess) {
        (void)hipStreamDestroy(g);
        return fail(UW_EHIP, "hipExtStreamCreateWithCUMask failed");
    }
    *gemm_stream = g;
    *decode_stream = dd;
    return UW_OK;
}

uw_status uw_stream_destroy(void* stream)
{
    using namespace uw;
    clear_error();
    if (!stream) return fail(UW_EINVAL, "NULL stream");
    if (hipStreamDestroy(static_cast<hipStream_t>(stream)) != hipSuccess) return fail(UW_EHIP, "hipStreamDestroy failed");
    return UW_OK;
}

uw_status uw_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, void* stream)
{
    using namespace uw;
    clear_error();
    if (!d_src || !d_sink) return fail(UW_EINVAL, "NULL argument");
    if (!aligned(d_src, 16) || bytes % 16 != 0) return fail(UW_EINVAL, "d_src and bytes must be multiples of 16");
    if (bytes == 0) return UW_OK;
    const uint32_t blocks = 8 * stream_cu_count(stream);
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(d_src), static_cast<uint64_t>(bytes / 16), d_sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(UW_EHIP, "stream read launch failed: %s", hipGetErrorString(e));
    return UW_OK;
}

uw_status uw_stream_cu_count(void* stream, int* out)
{
    using namespace uw;
    clear_error();
    if (!out) return fail(UW_EINVAL, "NULL output");
    *out = static_cast<int>(stream_cu_count(stream));
    return UW_OK;
}

}  // extern "C"
