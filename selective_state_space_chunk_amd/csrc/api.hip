// C ABI of libssd: argument validation, workspace carve-up and dispatch.
// Declarations and the contract of every entry point are in include/libssd.h.
#include "libssd.h"
#include "common.h"

#include <mutex>

#include <hip/hip_runtime.h>

namespace ssd {
hipError_t launch_staged_scan(const ScanArgs &a, const Workspace &ws);
bool mfma_supported(int64_t P, int64_t N, int64_t Q);
size_t gram_bytes(int64_t B, int64_t L, int64_t G, int64_t Q);
hipError_t launch_pipe_scan(const ScanArgs &a, const Workspace &ws);
bool pipe_supported(int64_t H, int64_t P, int64_t G, int64_t N);
bool block_prologue_supported(int64_t HP, int64_t GN, int64_t H, int64_t W);
hipError_t launch_block_prologue(const void *zx, const float *conv_w, const float *conv_b, const float *dt_bias,
                                 void *x, void *Bm, void *Cm, float *dt, int64_t B, int64_t L, int64_t H,
                                 int64_t HP, int64_t GN, int64_t W, hipStream_t stream);
bool gated_norm_supported(int64_t D, int64_t ngroups, int64_t zstride);
bool s6_supported(int64_t Dch, int64_t G, int64_t N);
hipError_t launch_s6(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                     const float *init, void *y, float *final_state, int64_t B, int64_t L, int64_t Dch, int64_t G,
                     int64_t N, int zoh, hipStream_t stream);
hipError_t launch_gated_norm(const void *y, const void *z, int64_t zstride, const float *w, const float *bias,
                             void *out, int64_t T, int64_t D, int64_t ngroups, float eps, int center,
                             hipStream_t stream);
bool bwd_supported(int64_t P, int64_t N, int64_t H, int64_t G);
size_t bwd_workspace_floats(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N);
hipError_t launch_scan_bwd(const void *x, const float *dt, const float *A, const void *Bm, const void *Cm,
                           const float *D, const float *init, const void *dy, const float *dfinal, void *dx,
                           float *ddt, float *dA, void *dBm, void *dCm, float *dD, float *dinit, float *ws,
                           int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, hipStream_t stream);
}

namespace {

using namespace ssd;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool pow2_in(int64_t v, int64_t lo, int64_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

bool shape_supported(int64_t P, int64_t N, int64_t Q) {
    return pow2_in(P, 16, 128) && pow2_in(N, 16, 256) && pow2_in(Q, 64, 256);
}

// Workspace regions of one call: only those the chosen kernels use.
struct Layout {
    size_t states, decay, seg, gram, total;
    size_t seg_floats;
};

// Most segment states the per-sequence scan keeps: it cuts sequences into at
// most as many segments as the device has compute units (256 on MI355X).
constexpr int64_t kSegStates = 256;

// Most (batch, head) sequences of one chunk-scan call.
constexpr int64_t kMaxChains = 65535;

// The algorithm a call runs: `algo` itself, or for SSD_ALGO_AUTO the
// per-sequence scan wherever it covers the shape (bfloat16, P = 64 or 128,
// N = 64, 128 or 256), else the staged matrix-core scan where it does
// (bfloat16, P = 64), else the float32 reference.  -1 when `algo` does not
// cover the shape or dtype.
int resolve(int64_t H, int64_t P, int64_t G, int64_t N, int64_t Q, ssd_dtype dtype, ssd_algo algo) {
    const bool bf16 = dtype == SSD_DTYPE_BF16;
    const bool staged_ok = bf16 && mfma_supported(P, N, Q);
    const bool pipe_ok = bf16 && pipe_supported(H, P, G, N);
    switch (algo) {
        case SSD_ALGO_AUTO:
            return pipe_ok ? SSD_ALGO_PIPE : staged_ok ? SSD_ALGO_STAGED : SSD_ALGO_REFERENCE;
        case SSD_ALGO_REFERENCE: return SSD_ALGO_REFERENCE;
        case SSD_ALGO_STAGED: return staged_ok ? SSD_ALGO_STAGED : -1;
        case SSD_ALGO_PIPE: return pipe_ok ? SSD_ALGO_PIPE : -1;
    }
    return -1;
}

// Byte offsets of each region for a resolved algorithm:
//  - reference and staged: the state of every block [B, nc, H, P, N] and its
//    decay [B, H, nc] (float32), and for staged the gram tiles of every block;
//  - per-sequence: the gram tiles of every 64-token sub-block and room for
//    the segment states (P*N floats and one log2 decay each) of the
//    sequences it cuts into time segments.
Layout layout(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t Q, int algo) {
    Layout l{};
    const int64_t nc = (L + Q - 1) / Q, nsb = (L + 63) / 64;
    size_t off = 0;
    if (algo == SSD_ALGO_REFERENCE || algo == SSD_ALGO_STAGED) {
        l.states = off; off = align_up(off + (size_t)(B * nc * H * P * N) * sizeof(float));
        l.decay = off;  off = align_up(off + (size_t)(B * H * nc) * sizeof(float));
    }
    if (algo == SSD_ALGO_STAGED) {
        l.gram = off; off = align_up(off + gram_bytes(B, L, G, Q));
    }
    if (algo == SSD_ALGO_PIPE) {
        // heads of 64 channels (a head of P = 128 is scanned as two)
        const int64_t cut = B * H * (P / 64) * (nsb > 1 ? nsb - 1 : 0);
        const int64_t nseg = cut < kSegStates ? cut : kSegStates;
        l.seg_floats = (size_t)(nseg * (64 * N + 1));
        l.seg = off;  off = align_up(off + l.seg_floats * sizeof(float));
        l.gram = off; off = align_up(off + gram_bytes(B, L, G, 64));
    }
    // never zero for a supported shape, so that a zero size means "not supported"
    l.total = off > 0 ? off : kAlign;
    return l;
}

Workspace carve(void *base, const Layout &l) {
    char *p = (char *)base;
    Workspace w;
    w.states = (float *)(p + l.states);
    w.decay = (float *)(p + l.decay);
    w.seg = (float *)(p + l.seg);
    w.seg_floats = l.seg_floats;
    w.gram = (void *)(p + l.gram);
    return w;
}

__global__ void fill_or_copy(float *__restrict__ dst, const float *__restrict__ src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// dt of packed rows with the reset flag in the sign bit: token t of row b is
// flagged when t > 0 and seq_idx changes there; every other dt keeps its
// magnitude with the sign bit clear.  A flat pass over the B*L*H values, VEC
// consecutive ones per thread (VEC = 4 when H % 4 == 0, so that a thread's
// values belong to one token and move as 16 bytes; else 1): 4.9 against
// 5.6 us at the 2.7B shape for one wave per token.
template <int VEC>
__global__ __launch_bounds__(256) void mark_resets(float *out, const float *dt, const int32_t *seq, int64_t L,
                                                   int64_t H, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VEC;
    if (i >= n) return;
    const int64_t bt = i / H;
    const bool reset = (bt % L) > 0 && seq[bt] != seq[bt - 1];
    const uint32_t flag = reset ? 0x80000000u : 0u;
    if constexpr (VEC == 4) {
        float4 v = *reinterpret_cast<const float4 *>(dt + i);
        v.x = __uint_as_float((__float_as_uint(v.x) & 0x7fffffffu) | flag);
        v.y = __uint_as_float((__float_as_uint(v.y) & 0x7fffffffu) | flag);
        v.z = __uint_as_float((__float_as_uint(v.z) & 0x7fffffffu) | flag);
        v.w = __uint_as_float((__float_as_uint(v.w) & 0x7fffffffu) | flag);
        *reinterpret_cast<float4 *>(out + i) = v;
    } else {
        out[i] = __uint_as_float((__float_as_uint(dt[i]) & 0x7fffffffu) | flag);
    }
}

// Plain streaming copy: one 16-byte chunk per thread, 4 KB per workgroup,
// non-temporal loads and stores (the shape that streamed fastest on MI355X:
// 6.6 TB/s read + written, against 6.1-6.3 TB/s with 16-32 KB per workgroup).
typedef unsigned copy_u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_copy(const copy_u32x4 *__restrict__ src,
                                                   copy_u32x4 *__restrict__ dst, int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

size_t varlen_extra(int64_t B, int64_t L, int64_t H) { return align_up((size_t)(B * L * H) * sizeof(float)); }

ssd_status common_checks(const void *x, const float *dt, const float *A, const void *Bm,
                         const void *Cm, const float *D, const void *y, int64_t B, int64_t L,
                         int64_t H, int64_t P, int64_t G, int64_t N, ssd_dtype dtype,
                         bool need_data) {
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0) return SSD_ERR_INVALID_ARG;
    if (H % G != 0) return SSD_ERR_INVALID_ARG;
    if (dtype != SSD_DTYPE_F32 && dtype != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (need_data) {
        if (!x || !dt || !A || !Bm || !Cm || !D || !y) return SSD_ERR_INVALID_ARG;
    }
    const void *ptrs[] = {x, dt, A, Bm, Cm, D, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_INVALID_ARG;
    return SSD_OK;
}

ssd_status scan_impl(const void *x, const float *dt, const float *A, const void *Bm, const void *Cm,
                     const float *D, const float *init, void *y, float *final_state,
                     void *workspace, size_t workspace_bytes, int64_t B, int64_t L, int64_t H,
                     int64_t P, int64_t G, int64_t N, int64_t Q, ssd_dtype dtype, ssd_algo algo,
                     hipStream_t stream) {
    const bool has_work = B > 0 && L > 0;
    ssd_status st = common_checks(x, dt, A, Bm, Cm, D, y, B, L, H, P, G, N, dtype, has_work);
    if (st != SSD_OK) return st;
    if ((init && !aligned16(init)) || (final_state && !aligned16(final_state)))
        return SSD_ERR_INVALID_ARG;
    if (Q <= 0) return SSD_ERR_INVALID_ARG;
    if (!shape_supported(P, N, Q)) return SSD_ERR_UNSUPPORTED;
    if (B > kMaxChains || H > kMaxChains || B * H > kMaxChains) return SSD_ERR_UNSUPPORTED;
    if ((L + Q - 1) / Q > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    const int run = resolve(H, P, G, N, Q, dtype, algo);
    if (run < 0) return SSD_ERR_UNSUPPORTED;
    const Layout l = layout(B, L, H, P, G, N, Q, run);
    if (has_work) {
        if (!workspace || workspace_bytes < l.total) return SSD_ERR_WORKSPACE;
        if (!aligned16(workspace)) return SSD_ERR_INVALID_ARG;
    }

    if (!has_work) {
        // nothing to scan: the final state is the initial state (or zeros)
        if (final_state && B > 0) {
            const int64_t n = B * H * P * N;
            if (init != final_state)
                fill_or_copy<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(final_state, init, n);
        }
        return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }

    ScanArgs a{x, dt, A, Bm, Cm, D, init, y, final_state, B, L, H, P, G, N, Q,
               dtype == SSD_DTYPE_BF16 ? 1 : 0, stream};
    const Workspace ws = carve(workspace, l);

    hipError_t e;
    switch (run) {
        case SSD_ALGO_REFERENCE: e = launch_reference_scan(a, ws); break;
        case SSD_ALGO_STAGED: e = launch_staged_scan(a, ws); break;
        case SSD_ALGO_PIPE: e = launch_pipe_scan(a, ws); break;
        default: return SSD_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

// Scratch of ssd_chunk_scan_fwd_noalloc: one array per device, created with
// the library's code object on that device and held until the process ends.
// Host code never uses the array's name as an address: the address on each
// device comes from hipGetSymbolAddress, once per device, with that device
// current.
__device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *ssd_status_string(ssd_status status) {
    switch (status) {
        case SSD_OK: return "SSD_OK";
        case SSD_ERR_INVALID_ARG: return "SSD_ERR_INVALID_ARG: invalid argument";
        case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape, chunk size, dtype or algorithm not supported";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
        case SSD_ERR_HIP: return "SSD_ERR_HIP: HIP runtime or launch failure";
        case SSD_ERR_TOO_LARGE:
            return "SSD_ERR_TOO_LARGE: the call needs more scratch than the no-allocation entry point holds";
    }
    return "unknown ssd_status";
}

const char *ssd_version(void) { return "libssd 0.1 (gfx950)"; }

size_t ssd_chunk_scan_workspace_size_algo(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                                          int64_t chunk_size, ssd_dtype dtype, ssd_algo algo) {
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || chunk_size <= 0) return 0;
    if (H % G != 0 || !shape_supported(P, N, chunk_size)) return 0;
    if (dtype != SSD_DTYPE_F32 && dtype != SSD_DTYPE_BF16) return 0;
    const int run = resolve(H, P, G, N, chunk_size, dtype, algo);
    if (run < 0) return 0;
    return layout(B, L, H, P, G, N, chunk_size, run).total;
}

size_t ssd_chunk_scan_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                     int64_t N, int64_t chunk_size, ssd_dtype dtype) {
    return ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, chunk_size, dtype, SSD_ALGO_AUTO);
}

ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A, const void *Bm,
                              const void *Cm, const float *D, const float *init_state, void *y,
                              float *final_state, void *workspace, size_t workspace_bytes,
                              int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                              int64_t chunk_size, ssd_dtype dtype, hipStream_t stream) {
    return scan_impl(x, dt, A, Bm, Cm, D, init_state, y, final_state, workspace, workspace_bytes,
                     B, L, H, P, G, N, chunk_size, dtype, SSD_ALGO_AUTO, stream);
}

ssd_status ssd_chunk_scan_fwd_algo(const void *x, const float *dt, const float *A, const void *Bm,
                                   const void *Cm, const float *D, const float *init_state, void *y,
                                   float *final_state, void *workspace, size_t workspace_bytes,
                                   int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                                   int64_t chunk_size, ssd_dtype dtype, ssd_algo algo,
                                   hipStream_t stream) {
    return scan_impl(x, dt, A, Bm, Cm, D, init_state, y, final_state, workspace, workspace_bytes,
                     B, L, H, P, G, N, chunk_size, dtype, algo, stream);
}

ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A, const void *Bm,
                                      const void *Cm, const float *D, const float *init_state, void *y,
                                      float *final_state, int64_t B, int64_t L, int64_t H, int64_t P,
                                      int64_t G, int64_t N, int64_t chunk_size, ssd_dtype dtype,
                                      hipStream_t stream) {
    const size_t need = ssd_chunk_scan_workspace_size(B, L, H, P, G, N, chunk_size, dtype);
    if (need > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_TOO_LARGE;
    // need == 0 (a shape outside the support matrix): scan_impl reports why
    void *ws = nullptr;
    if (need > 0 && B > 0 && L > 0 && scratch_address(&ws) != hipSuccess) return SSD_ERR_HIP;
    return scan_impl(x, dt, A, Bm, Cm, D, init_state, y, final_state, ws, ws ? SSD_NOALLOC_SCRATCH_BYTES : 0,
                     B, L, H, P, G, N, chunk_size, dtype, SSD_ALGO_AUTO, stream);
}

size_t ssd_chunk_scan_varlen_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                            int64_t N, int64_t chunk_size, ssd_dtype dtype) {
    if (dtype != SSD_DTYPE_BF16 || N > 128) return 0;
    const size_t base = ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, chunk_size, dtype, SSD_ALGO_PIPE);
    if (base == 0) return 0;
    return align_up(base) + varlen_extra(B, L, H);
}

ssd_status ssd_chunk_scan_fwd_varlen(const void *x, const float *dt, const float *A, const void *Bm,
                                     const void *Cm, const float *D, const float *init_state,
                                     const int32_t *seq_idx, void *y, float *final_state,
                                     void *workspace, size_t workspace_bytes, int64_t B, int64_t L,
                                     int64_t H, int64_t P, int64_t G, int64_t N, int64_t chunk_size,
                                     ssd_dtype dtype, hipStream_t stream) {
    const bool has_work = B > 0 && L > 0;
    ssd_status st = common_checks(x, dt, A, Bm, Cm, D, y, B, L, H, P, G, N, dtype, has_work);
    if (st != SSD_OK) return st;
    if ((init_state && !aligned16(init_state)) || (final_state && !aligned16(final_state)))
        return SSD_ERR_INVALID_ARG;
    if (has_work && !seq_idx) return SSD_ERR_INVALID_ARG;
    if (((uintptr_t)seq_idx & 3u) != 0) return SSD_ERR_INVALID_ARG;
    if (chunk_size <= 0) return SSD_ERR_INVALID_ARG;
    if (!shape_supported(P, N, chunk_size) || dtype != SSD_DTYPE_BF16 || !pipe_supported(H, P, G, N) || N > 128)
        return SSD_ERR_UNSUPPORTED;
    if (B > kMaxChains || H > kMaxChains || B * H > kMaxChains) return SSD_ERR_UNSUPPORTED;
    if ((L + chunk_size - 1) / chunk_size > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    if (!has_work)
        return scan_impl(x, dt, A, Bm, Cm, D, init_state, y, final_state, workspace, workspace_bytes, B, L, H, P, G,
                         N, chunk_size, dtype, SSD_ALGO_PIPE, stream);
    const Layout l = layout(B, L, H, P, G, N, chunk_size, SSD_ALGO_PIPE);
    const size_t base = align_up(l.total);
    if (!workspace || workspace_bytes < base + varlen_extra(B, L, H)) return SSD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SSD_ERR_INVALID_ARG;
    float *marked = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + base);
    const int64_t nval = B * L * H;
    const int vec = H % 4 == 0 && aligned16(dt) ? 4 : 1;
    const int64_t nwg = (nval / vec + 255) / 256;
    if (nwg > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    if (vec == 4)
        mark_resets<4><<<(unsigned)nwg, 256, 0, stream>>>(marked, dt, seq_idx, L, H, nval);
    else
        mark_resets<1><<<(unsigned)nwg, 256, 0, stream>>>(marked, dt, seq_idx, L, H, nval);
    if (hipGetLastError() != hipSuccess) return SSD_ERR_HIP;
    ScanArgs a{x, marked, A, Bm, Cm, D, init_state, y, final_state, B, L, H, P, G, N, chunk_size, 1, stream, 1};
    const hipError_t e = launch_pipe_scan(a, carve(workspace, l));
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_block_prologue(const void *zxbcdt, const float *conv_w, const float *conv_b,
                              const float *dt_bias, void *x, void *Bm, void *Cm, float *dt, int64_t B,
                              int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t W,
                              ssd_dtype dtype, hipStream_t stream) {
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || W <= 0) return SSD_ERR_INVALID_ARG;
    if (H % G != 0) return SSD_ERR_INVALID_ARG;
    if (dtype != SSD_DTYPE_BF16 || !block_prologue_supported(H * P, G * N, H, W)) return SSD_ERR_UNSUPPORTED;
    if (B == 0 || L == 0) return SSD_OK;
    if (!zxbcdt || !conv_w || !x || !Bm || !Cm || !dt) return SSD_ERR_INVALID_ARG;
    const void *ptrs[] = {zxbcdt, x, Bm, Cm};
    for (const void *p : ptrs)
        if (!aligned16(p)) return SSD_ERR_INVALID_ARG;
    if ((L + 127) / 128 > 65535 || B > 65535) return SSD_ERR_UNSUPPORTED;   // the prologue grid: 128-token tiles
    const hipError_t e = launch_block_prologue(zxbcdt, conv_w, conv_b, dt_bias, x, Bm, Cm, dt, B, L, H, H * P,
                                               G * N, W, stream);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_gated_norm(const void *y, const void *z, int64_t z_stride, const float *weight, const float *bias,
                          void *out, int64_t T, int64_t D, int64_t ngroups, float eps, int center,
                          ssd_dtype dtype, hipStream_t stream) {
    if (T < 0 || D <= 0 || ngroups <= 0 || !(eps >= 0.f)) return SSD_ERR_INVALID_ARG;
    if (dtype != SSD_DTYPE_BF16 || !gated_norm_supported(D, ngroups, z_stride)) return SSD_ERR_UNSUPPORTED;
    if (T == 0) return SSD_OK;
    if (!y || !z || !weight || !out) return SSD_ERR_INVALID_ARG;
    const void *ptrs[] = {y, z, out};
    for (const void *p : ptrs)
        if (!aligned16(p)) return SSD_ERR_INVALID_ARG;
    if ((T + 3) / 4 > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    if (((uintptr_t)weight & 15u) != 0 || ((uintptr_t)bias & 15u) != 0) return SSD_ERR_INVALID_ARG;
    const hipError_t e = launch_gated_norm(y, z, z_stride, weight, bias, out, T, D, ngroups, eps, center, stream);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_selective_scan(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm,
                              const float *D, const float *init_state, void *y, float *final_state, int64_t B,
                              int64_t L, int64_t Dch, int64_t G, int64_t N, int zoh, ssd_dtype dtype,
                              hipStream_t stream) {
    if (B < 0 || L < 0 || Dch <= 0 || G <= 0 || N <= 0 || Dch % G != 0) return SSD_ERR_INVALID_ARG;
    if (dtype != SSD_DTYPE_BF16 || !s6_supported(Dch, G, N)) return SSD_ERR_UNSUPPORTED;
    if (B > 65535 || Dch / 64 > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    if (B == 0) return SSD_OK;
    if (L == 0) {
        if (final_state) {
            const int64_t n = B * Dch * N;
            if (init_state != final_state)
                fill_or_copy<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(final_state, init_state, n);
        }
        return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
    if (!x || !dt || !A || !Bm || !Cm || !y) return SSD_ERR_INVALID_ARG;
    const void *ptrs[] = {x, dt, Bm, Cm, y};
    for (const void *p : ptrs)
        if (!aligned16(p)) return SSD_ERR_INVALID_ARG;
    const hipError_t e = launch_s6(x, dt, A, Bm, Cm, D, init_state, y, final_state, B, L, Dch, G, N, zoh, stream);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

size_t ssd_chunk_scan_bwd_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                         int64_t N, int64_t chunk_size, ssd_dtype dtype) {
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || chunk_size <= 0) return 0;
    if (H % G != 0 || !shape_supported(P, N, chunk_size)) return 0;
    if (dtype != SSD_DTYPE_BF16 || !bwd_supported(P, N, H, G)) return 0;
    return align_up(bwd_workspace_floats(B, L, H, P, N) * sizeof(float));
}

ssd_status ssd_chunk_scan_bwd(const void *x, const float *dt, const float *A, const void *Bm,
                              const void *Cm, const float *D, const float *init_state, const void *dy,
                              const float *dfinal, void *dx, float *ddt, float *dA, void *dBm, void *dCm,
                              float *dD, float *dinit, void *workspace, size_t workspace_bytes, int64_t B,
                              int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t chunk_size,
                              ssd_dtype dtype, hipStream_t stream) {
    const bool has_work = B > 0 && L > 0;
    ssd_status st = common_checks(x, dt, A, Bm, Cm, D, dy, B, L, H, P, G, N, dtype, has_work);
    if (st != SSD_OK) return st;
    if (!dA || !dD) return SSD_ERR_INVALID_ARG;
    if (has_work && (!dx || !ddt || !dBm || !dCm)) return SSD_ERR_INVALID_ARG;
    const void *ptrs[] = {init_state, dfinal, dx, ddt, dA, dBm, dCm, dD, dinit};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return SSD_ERR_INVALID_ARG;
    if (chunk_size <= 0) return SSD_ERR_INVALID_ARG;
    if (!shape_supported(P, N, chunk_size) || dtype != SSD_DTYPE_BF16 || !bwd_supported(P, N, H, G))
        return SSD_ERR_UNSUPPORTED;
    const int64_t Hk = H * (P / 64);   // heads of 64 channels
    if (B > kMaxChains || Hk > kMaxChains || B * Hk > kMaxChains) return SSD_ERR_UNSUPPORTED;
    const int64_t nsb = (L + 63) / 64;
    if (B * Hk * nsb > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    if (!has_work) {
        // no tokens: dA = dD = 0 and the initial state's gradient is dfinal (or 0)
        fill_or_copy<<<(unsigned)((H + 255) / 256), 256, 0, stream>>>(dA, nullptr, H);
        fill_or_copy<<<(unsigned)((H + 255) / 256), 256, 0, stream>>>(dD, nullptr, H);
        if (dinit && B > 0) {
            const int64_t n = B * H * P * N;
            fill_or_copy<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(dinit, dfinal, n);
        }
        return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
    const size_t need = align_up(bwd_workspace_floats(B, L, H, P, N) * sizeof(float));
    if (!workspace || workspace_bytes < need) return SSD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SSD_ERR_INVALID_ARG;
    const hipError_t e = launch_scan_bwd(x, dt, A, Bm, Cm, D, init_state, dy, dfinal, dx, ddt, dA, dBm, dCm,
                                         dD, dinit, (float *)workspace, B, L, H, P, G, N, stream);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return SSD_OK;
    if (!dst || !src || !aligned16(dst) || !aligned16(src) || bytes % 16 != 0) return SSD_ERR_INVALID_ARG;
    const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
    if (d < s + bytes && s < d + bytes) return SSD_ERR_INVALID_ARG;   // overlapping
    const int64_t n16 = (int64_t)(bytes / 16);
    if ((n16 + 255) / 256 > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    stream_copy<<<(unsigned)((n16 + 255) / 256), 256, 0, stream>>>((const copy_u32x4 *)src, (copy_u32x4 *)dst, n16);
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_step(float *state, const void *x, const float *dt, const float *A, const void *Bm,
                    const void *Cm, const float *D, void *y, int64_t B, int64_t H, int64_t P,
                    int64_t G, int64_t N, ssd_dtype dtype, hipStream_t stream) {
    ssd_status st = common_checks(x, dt, A, Bm, Cm, D, y, B, 1, H, P, G, N, dtype, B > 0);
    if (st != SSD_OK) return st;
    if (B > 0 && !state) return SSD_ERR_INVALID_ARG;
    if (state && !aligned16(state)) return SSD_ERR_INVALID_ARG;
    if (!pow2_in(P, 16, 128) || !pow2_in(N, 16, 256)) return SSD_ERR_UNSUPPORTED;
    if (B * H > 0x7fffffff / 32) return SSD_ERR_UNSUPPORTED;   // up to 32 workgroups per (b, h)
    if (B == 0) return SSD_OK;
    const hipError_t e = launch_step(state, x, dt, A, Bm, Cm, D, y, B, H, P, G, N,
                                     dtype == SSD_DTYPE_BF16 ? 1 : 0, stream);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
