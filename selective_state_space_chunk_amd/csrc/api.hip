// C ABI of libssd: argument validation, workspace carve-up and dispatch.
// Declarations and the contract of every entry point are in include/libssd.h.
#include "libssd.h"
#include "common.h"

#include <vector>

#include <hip/hip_runtime.h>

namespace ssd {
hipError_t launch_staged_scan(const ScanArgs &a, const Workspace &ws);
hipError_t launch_fused_scan(const ScanArgs &a, const Workspace &ws);
bool mfma_supported(int64_t P, int64_t N, int64_t Q);
size_t gram_bytes(int64_t B, int64_t L, int64_t G, int64_t Q);
bool fused_supported(int64_t H, int64_t G, int64_t N, int64_t Q);
hipError_t launch_chain_scan(const ScanArgs &a, const Workspace &ws);
bool chain_supported(int64_t H, int64_t G, int64_t N);
hipError_t launch_pipe_scan(const ScanArgs &a, const Workspace &ws);
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
bool pipe_supported(int64_t H, int64_t G, int64_t N);
hipError_t launch_pair_scan(const ScanArgs &a, const Workspace &ws);
bool pair_supported(int64_t H, int64_t G, int64_t N);
bool bwd_supported(int64_t P, int64_t N, int64_t H, int64_t G);
size_t bwd_workspace_floats(int64_t B, int64_t L, int64_t H, int64_t N);
hipError_t launch_scan_bwd(const void *x, const float *dt, const float *A, const void *Bm, const void *Cm,
                           const float *D, const float *init, const void *dy, const float *dfinal, void *dx,
                           float *ddt, float *dA, void *dBm, void *dCm, float *dD, float *dinit, float *ws,
                           int64_t B, int64_t L, int64_t H, int64_t G, int64_t N, hipStream_t stream);
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

struct Layout {
    size_t states, decay, flags, counters, ring, gram, total;
    size_t ring_floats;
};

// Segment states the workspace holds for the per-sequence scan.
constexpr int64_t kSegStates = 256;

// Most (batch, head) chains the hand-off flags cover; scans are limited to it.
constexpr int64_t kMaxChains = 65535;

// Byte offsets of each workspace region.  The counters and flags sit at the
// same offsets for every shape, ahead of all scratch, so that they are never
// overwritten by another call's scratch and stay zero between calls.
Layout layout(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t Q) {
    Layout l{};
    const int64_t nc = (L + Q - 1) / Q;
    size_t off = 0;
    l.counters = off; off = align_up(off + 4 * sizeof(unsigned));
    l.flags = off;    off = align_up(off + (size_t)kMaxChains * sizeof(unsigned));
    l.states = off;   off = align_up(off + (size_t)(B * nc * H * P * N) * sizeof(float));
    l.decay = off;    off = align_up(off + (size_t)(B * H * nc) * sizeof(float));
    // the ring also holds the segment states of the per-sequence matrix-core
    // scan (P = 64, N <= 128): room for 256 of them, one per compute unit
    const int64_t seg_floats = (P == 64 && (N == 64 || N == 128)) ? kSegStates * (P * N + 1) : 0;
    const int64_t ring_floats = B * H * 2 * P * N > seg_floats ? B * H * 2 * P * N : seg_floats;
    l.ring = off;     off = align_up(off + (size_t)ring_floats * sizeof(float));
    l.ring_floats = (size_t)ring_floats;
    l.gram = off;     off = align_up(off + gram_bytes(B, L, G, Q));
    l.total = off;
    return l;
}

Workspace carve(void *base, const Layout &l) {
    char *p = (char *)base;
    Workspace w;
    w.states = (float *)(p + l.states);
    w.decay = (float *)(p + l.decay);
    w.flags = (unsigned *)(p + l.flags);
    w.counters = (unsigned *)(p + l.counters);
    w.ring = (float *)(p + l.ring);
    w.ring_floats = l.ring_floats;
    w.gram = (void *)(p + l.gram);
    return w;
}

__global__ void fill_or_copy(float *__restrict__ dst, const float *__restrict__ src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// dt of packed rows with the reset flag in the sign bit: token t of row b is
// flagged when t > 0 and seq_idx changes there; every other dt keeps its
// magnitude with the sign bit clear.  One wave per token (b, t) of the B*L,
// its lanes over the H heads.
__global__ __launch_bounds__(256) void mark_resets(float *out, const float *dt, const int32_t *seq, int64_t L,
                                                   int64_t H, int64_t ntok) {
    const int64_t bt = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (bt >= ntok) return;
    const bool reset = (bt % L) > 0 && seq[bt] != seq[bt - 1];
    const uint32_t flag = reset ? 0x80000000u : 0u;
    const float *src = dt + bt * H;
    float *dst = out + bt * H;
    for (int64_t h = threadIdx.x & 63; h < H; h += 64)
        dst[h] = __uint_as_float((__float_as_uint(src[h]) & 0x7fffffffu) | flag);
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
    if (algo != SSD_ALGO_AUTO && algo != SSD_ALGO_REFERENCE && algo != SSD_ALGO_STAGED &&
        algo != SSD_ALGO_FUSED && algo != SSD_ALGO_CHAIN && algo != SSD_ALGO_PIPE && algo != SSD_ALGO_PAIR)
        return SSD_ERR_UNSUPPORTED;
    const bool mfma_ok = dtype == SSD_DTYPE_BF16 && mfma_supported(P, N, Q);
    if ((algo == SSD_ALGO_STAGED || algo == SSD_ALGO_FUSED || algo == SSD_ALGO_CHAIN || algo == SSD_ALGO_PIPE ||
         algo == SSD_ALGO_PAIR) &&
        !mfma_ok)
        return SSD_ERR_UNSUPPORTED;
    if (algo == SSD_ALGO_CHAIN && !chain_supported(H, G, N)) return SSD_ERR_UNSUPPORTED;
    if (algo == SSD_ALGO_PIPE && !pipe_supported(H, G, N)) return SSD_ERR_UNSUPPORTED;
    if (algo == SSD_ALGO_PAIR && !pair_supported(H, G, N)) return SSD_ERR_UNSUPPORTED;
    if (algo == SSD_ALGO_FUSED && !fused_supported(H, G, N, Q)) return SSD_ERR_UNSUPPORTED;
    if (algo == SSD_ALGO_FUSED && B * H * ((L + Q - 1) / Q) > 0x7fffffff) return SSD_ERR_UNSUPPORTED;

    const Layout l = layout(B, L, H, P, G, N, Q);
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

    if (algo == SSD_ALGO_AUTO) {
        if (!mfma_ok) {
            algo = SSD_ALGO_REFERENCE;
        } else {
            const int64_t nc = (L + Q - 1) / Q;
            // per-sequence scan (spread over the device in time segments when
            // sequences are few) wherever it covers the shape; else one pass
            // while chains of blocks are short and many; staged otherwise
            if (pipe_supported(H, G, N))
                algo = SSD_ALGO_PIPE;
            else
                algo = (nc <= 64 && fused_supported(H, G, N, Q) && B * H >= 64 && B * H * nc <= 0x7fffffff)
                           ? SSD_ALGO_FUSED : SSD_ALGO_STAGED;
        }
    }
    hipError_t e;
    switch (algo) {
        case SSD_ALGO_REFERENCE: e = launch_reference_scan(a, ws); break;
        case SSD_ALGO_STAGED: e = launch_staged_scan(a, ws); break;
        case SSD_ALGO_FUSED: e = launch_fused_scan(a, ws); break;
        case SSD_ALGO_CHAIN: e = launch_chain_scan(a, ws); break;
        case SSD_ALGO_PIPE: e = launch_pipe_scan(a, ws); break;
        case SSD_ALGO_PAIR: e = launch_pair_scan(a, ws); break;
        default: return SSD_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
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
    }
    return "unknown ssd_status";
}

const char *ssd_version(void) { return "libssd 0.1 (gfx950)"; }

size_t ssd_chunk_scan_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                     int64_t N, int64_t chunk_size, ssd_dtype dtype) {
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || chunk_size <= 0) return 0;
    if (H % G != 0 || !shape_supported(P, N, chunk_size)) return 0;
    if (dtype != SSD_DTYPE_F32 && dtype != SSD_DTYPE_BF16) return 0;
    return layout(B, L, H, P, G, N, chunk_size).total;
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

size_t ssd_chunk_scan_varlen_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                            int64_t N, int64_t chunk_size, ssd_dtype dtype) {
    const size_t base = ssd_chunk_scan_workspace_size(B, L, H, P, G, N, chunk_size, dtype);
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
    if (!shape_supported(P, N, chunk_size) || dtype != SSD_DTYPE_BF16 || !mfma_supported(P, N, chunk_size) ||
        !pipe_supported(H, G, N))
        return SSD_ERR_UNSUPPORTED;
    if (B > kMaxChains || H > kMaxChains || B * H > kMaxChains) return SSD_ERR_UNSUPPORTED;
    if ((L + chunk_size - 1) / chunk_size > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    if (!has_work)
        return scan_impl(x, dt, A, Bm, Cm, D, init_state, y, final_state, workspace, workspace_bytes, B, L, H, P, G,
                         N, chunk_size, dtype, SSD_ALGO_PIPE, stream);
    const Layout l = layout(B, L, H, P, G, N, chunk_size);
    const size_t base = align_up(l.total);
    if (!workspace || workspace_bytes < base + varlen_extra(B, L, H)) return SSD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SSD_ERR_INVALID_ARG;
    float *marked = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + base);
    const int64_t ntok = B * L;
    if ((ntok + 3) / 4 > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    mark_resets<<<(unsigned)((ntok + 3) / 4), 256, 0, stream>>>(marked, dt, seq_idx, L, H, ntok);
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
    if ((L + 31) / 32 > 65535 || B > 65535) return SSD_ERR_UNSUPPORTED;
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
    return align_up(bwd_workspace_floats(B, L, H, N) * sizeof(float));
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
    if (B > kMaxChains || H > kMaxChains || B * H > kMaxChains) return SSD_ERR_UNSUPPORTED;
    const int64_t nsb = (L + 63) / 64;
    if (B * H * nsb > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
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
    const size_t need = align_up(bwd_workspace_floats(B, L, H, N) * sizeof(float));
    if (!workspace || workspace_bytes < need) return SSD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SSD_ERR_INVALID_ARG;
    const hipError_t e = launch_scan_bwd(x, dt, A, Bm, Cm, D, init_state, dy, dfinal, dx, ddt, dA, dBm, dCm,
                                         dD, dinit, (float *)workspace, B, L, H, G, N, stream);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status ssd_chunk_scan_workspace_check(void *workspace, size_t workspace_bytes, int64_t B,
                                          int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                                          int64_t chunk_size, hipStream_t stream) {
    if (!workspace || B < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || chunk_size <= 0)
        return SSD_ERR_INVALID_ARG;
    const Layout l = layout(B, L, H, P, G, N, chunk_size);
    if (workspace_bytes < l.total) return SSD_ERR_WORKSPACE;
    unsigned *ctr = (unsigned *)((char *)workspace + l.counters);
    unsigned host[4] = {0, 0, 0, 0};
    if (hipStreamSynchronize(stream) != hipSuccess) return SSD_ERR_HIP;
    if (hipMemcpy(host, ctr, sizeof(host), hipMemcpyDeviceToHost) != hipSuccess) return SSD_ERR_HIP;
    if (host[2] != 0) {
        const unsigned zero = 0;
        if (hipMemcpy(ctr + 2, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return SSD_ERR_HIP;
        return SSD_ERR_HIP;
    }
    if (host[0] != 0 || host[1] != 0) return SSD_ERR_HIP;
    const int64_t chains = B * H < kMaxChains ? B * H : kMaxChains;
    if (chains > 0) {
        std::vector<unsigned> flags((size_t)chains);
        if (hipMemcpy(flags.data(), (char *)workspace + l.flags, flags.size() * sizeof(unsigned),
                      hipMemcpyDeviceToHost) != hipSuccess)
            return SSD_ERR_HIP;
        for (unsigned f : flags)
            if (f != 0) return SSD_ERR_HIP;
    }
    return SSD_OK;
}

ssd_status ssd_step(float *state, const void *x, const float *dt, const float *A, const void *Bm,
                    const void *Cm, const float *D, void *y, int64_t B, int64_t H, int64_t P,
                    int64_t G, int64_t N, ssd_dtype dtype, hipStream_t stream) {
    ssd_status st = common_checks(x, dt, A, Bm, Cm, D, y, B, 1, H, P, G, N, dtype, B > 0);
    if (st != SSD_OK) return st;
    if (B > 0 && !state) return SSD_ERR_INVALID_ARG;
    if (state && !aligned16(state)) return SSD_ERR_INVALID_ARG;
    if (!pow2_in(P, 16, 128) || !pow2_in(N, 16, 256)) return SSD_ERR_UNSUPPORTED;
    if (B * H > 0x7fffffff) return SSD_ERR_UNSUPPORTED;
    if (B == 0) return SSD_OK;
    const hipError_t e = launch_step(state, x, dt, A, Bm, Cm, D, y, B, H, P, G, N,
                                     dtype == SSD_DTYPE_BF16 ? 1 : 0, stream);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
