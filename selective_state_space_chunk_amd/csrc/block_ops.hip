// The steps on either side of the scan in a Mamba-2 block (the "Mamba-2"
// note, section "Mamba-2 block": one parallel projection gives the gate input
// z, X, B, C and the step dt; the scan output is gated and normalised before
// the output projection, a GroupNorm per the "Mamba-2" walkthrough, section
// 7.2).  Both kernels stream HBM once: every value is read once and every
// output written once, 16 bytes per lane, with the work of a token or a tile
// of tokens kept in registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

namespace {

typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x8 ld_bf16x8(const __bf16 *p) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    f32x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
    return v;
}
// 16 bytes read once (non-temporal: they need not stay in the caches)
__device__ __forceinline__ uint4 ld_stream(const __bf16 *p) {
    typedef unsigned int u32x4n __attribute__((ext_vector_type(4)));
    const u32x4n v = __builtin_nontemporal_load(reinterpret_cast<const u32x4n *>(p));
    return uint4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void st_bf16x8(__bf16 *p, const f32x8 &v) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    bf16x8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)v[e];
    *reinterpret_cast<bf16x8_t *>(p) = o;
}
// v * logistic(v) with the hardware reciprocal (about 1 ulp; the outputs are
// rounded to bfloat16); v far below zero gives exp = inf, reciprocal 0, -0
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }
__device__ __forceinline__ float softplus(float v) { return v > 20.f ? v : log1pf(__expf(v)); }

// ---------------------------------------------------------------------------
// Prologue.  Projection row of a token: [z (HP) | x (HP) | Bm (GN) | Cm (GN) |
// dt (H)], bfloat16.  The C = HP + 2GN middle channels go through a causal
// depthwise convolution of width W (taps conv_w[c][k], tap W-1 on the
// current token, zero before token 0) plus bias and SiLU, into x, Bm, Cm;
// dt = softplus(dt_raw + dt_bias).  Workgroup (ty, cx, b): 128 tokens of row
// b from token 128 ty; lane k of channel tile cx takes channels 8(256 cx + k)
// .. +7 for all 128 tokens, keeping the last W-1 inputs in registers and
// loading the next 4 rows while the current 4 are computed.  The last channel
// tile computes dt of the 128 tokens instead.  At the 2.7B layer shape 128
// tokens per workgroup took 94 us, against 112 us with 32 (whose workgroups
// re-read 3 of every 32 rows for the convolution's history) and 120 us with
// 256; loading ahead took it to 92 us.  The rows are read once, so they are
// loaded non-temporally (83 against 89 us), and rounds of 4 rows instead of 8
// hold 120 registers instead of 193 (81 against 83 us).
struct ProArgs {
    const __bf16 *zx;
    const float *conv_w, *conv_b, *dt_bias;
    __bf16 *x, *Bm, *Cm;
    float *dt;
    int64_t L, HP, GN, H, row;
    int ctiles;
};

constexpr int kTok = 128;

template <int W>
__global__ __launch_bounds__(256) void prologue_kernel(ProArgs a) {
    const int64_t b = blockIdx.z;
    const int64_t t0 = (int64_t)blockIdx.x * kTok;
    const int nt = (int)(a.L - t0 < kTok ? a.L - t0 : kTok);
    const __bf16 *rows = a.zx + (b * a.L) * a.row;
    if ((int)blockIdx.y == a.ctiles) {
        const int H = (int)a.H;
        const int64_t off = 2 * a.HP + 2 * a.GN;
        for (int i = threadIdx.x; i < nt * H; i += 256) {
            const int tt = i / H, h = i - tt * H;
            const float v = (float)rows[(t0 + tt) * a.row + off + h] + (a.dt_bias ? a.dt_bias[h] : 0.f);
            a.dt[(b * a.L + t0 + tt) * a.H + h] = softplus(v);
        }
        return;
    }
    const int64_t C = a.HP + 2 * a.GN;
    const int64_t c = 8 * ((int64_t)blockIdx.y * 256 + threadIdx.x);
    if (c >= C) return;
    float wk[W][8], bias[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bias[e] = a.conv_b ? a.conv_b[c + e] : 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k][e] = a.conv_w[(c + e) * W + k];
    }
    const __bf16 *src = rows + a.HP + c;
    // destination of these channels
    __bf16 *dst;
    int64_t dstride;
    if (c < a.HP) {
        dst = a.x + b * a.L * a.HP + c;
        dstride = a.HP;
    } else if (c < a.HP + a.GN) {
        dst = a.Bm + b * a.L * a.GN + (c - a.HP);
        dstride = a.GN;
    } else {
        dst = a.Cm + b * a.L * a.GN + (c - a.HP - a.GN);
        dstride = a.GN;
    }
    // rows are kept as raw bfloat16 words and widened where they are used
    constexpr int R = 4;   // tokens per round: their loads go out together
    uint4 hist[W > 1 ? W - 1 : 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t t = t0 - (W - 1) + j;
        hist[j] = t >= 0 ? ld_stream(src + t * a.row) : uint4{0u, 0u, 0u, 0u};
    }
    auto widen = [](const uint4 &u, int e) {
        const uint32_t w = e < 2 ? (e == 0 ? u.x : u.y) : (e == 2 ? u.z : u.w);
        return w;
    };
    uint4 nxt[R];   // the rows of the next round
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int t = u < nt ? u : nt - 1;   // clamped: every load in bounds
        nxt[u] = ld_stream(src + (t0 + t) * a.row);
    }
    for (int tt = 0; tt < nt; tt += R) {
        uint4 cur[R];
#pragma unroll
        for (int u = 0; u < R; ++u) cur[u] = nxt[u];
        if (tt + R < nt) {
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int t = tt + R + u < nt ? tt + R + u : nt - 1;   // clamped: every load in bounds
                nxt[u] = ld_stream(src + (t0 + t) * a.row);
            }
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            f32x8 acc;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                auto val = [&](const uint4 &r) {
                    const uint32_t w = widen(r, e >> 1);
                    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
                };
                float s = bias[e];
#pragma unroll
                for (int k = 0; k < W - 1; ++k) s = __builtin_fmaf(wk[k][e], val(hist[k]), s);
                acc[e] = silu(__builtin_fmaf(wk[W - 1][e], val(cur[u]), s));
            }
            if (tt + u < nt) st_bf16x8(dst + (t0 + tt + u) * dstride, acc);
#pragma unroll
            for (int j = 0; j + 1 < W - 1; ++j) hist[j] = hist[j + 1];
            if constexpr (W > 1) hist[W - 2] = cur[u];
        }
    }
}

// ---------------------------------------------------------------------------
// Gated norm.  One wave per token (four tokens per workgroup): v = y * SiLU(z)
// over its D channels, normalised within each of ngroups equal groups
// (mean-centred with variance, or root mean square only), times weight, plus
// bias.  Lane l holds channel chunks l, l + 64, ... (8 channels each, KC
// chunks) in registers, so that all of a token's loads are in flight at once
// and the group sums are wave reductions with no barrier.  The loaded y and z
// stay raw bfloat16 words until used: 122 registers instead of 185 at D =
// 5120, four waves per SIMD instead of two (110 against 125 us at the 2.7B
// layer shape), and are loaded non-temporally (98 against 109 us).  The sums
// run in a fixed order, so results are deterministic.
struct NormArgs {
    const __bf16 *y, *z;
    const float *w, *bias;
    __bf16 *out;
    int64_t T, D, zstride;
    int ngroups, center;
    float eps;
};

constexpr int kMaxGroups = 8;

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// tot[g] = sum over the wave of part[k] for this lane's chunks of group g
template <int KC>
__device__ __forceinline__ void group_sums(const float (&part)[KC], const int (&grp)[KC], int ngroups,
                                           float (&tot)[kMaxGroups]) {
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g) {
        tot[g] = 0.f;
        if (g < ngroups) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < KC; ++k) s += grp[k] == g ? part[k] : 0.f;
            tot[g] = wave_sum64(s);
        }
    }
}

template <int KC>
__global__ __launch_bounds__(256) void gated_norm_kernel(NormArgs a) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int lane = threadIdx.x & 63;
    const int nch = (int)(a.D / 8), gch = nch / a.ngroups;
    const float inv = 1.f / (float)(a.D / a.ngroups);
    // y and z stay raw bfloat16 words until used (half the registers of
    // widened values: more waves per SIMD to keep loads in flight)
    uint4 yr[KC], zr[KC];
    int grp[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int ch = lane + 64 * k;
        grp[k] = ch < nch ? ch / gch : -1;
        const int cl = ch < nch ? ch : nch - 1;   // clamped: every load in bounds
        yr[k] = ld_stream(a.y + t * a.D + 8 * cl);
        zr[k] = ld_stream(a.z + t * a.zstride + 8 * cl);
    }
    f32x8 v[KC];
    float part[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        part[k] = 0.f;
        const uint32_t yw[4] = {yr[k].x, yr[k].y, yr[k].z, yr[k].w};
        const uint32_t zw[4] = {zr[k].x, zr[k].y, zr[k].z, zr[k].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float yy = __uint_as_float((e & 1) ? (yw[e >> 1] & 0xffff0000u) : (yw[e >> 1] << 16));
            const float zz = __uint_as_float((e & 1) ? (zw[e >> 1] & 0xffff0000u) : (zw[e >> 1] << 16));
            v[k][e] = yy * silu(zz);
            part[k] += v[k][e];
        }
    }
    float tot[kMaxGroups];
    if (a.center) {
        group_sums<KC>(part, grp, a.ngroups, tot);
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            float m = 0.f;
#pragma unroll
            for (int g = 0; g < kMaxGroups; ++g) m = g == grp[k] ? tot[g] * inv : m;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[k][e] -= m;
        }
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        part[k] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part[k] = __builtin_fmaf(v[k][e], v[k][e], part[k]);
    }
    group_sums<KC>(part, grp, a.ngroups, tot);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        if (grp[k] < 0) continue;
        float ms = 0.f;
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g) ms = g == grp[k] ? tot[g] : ms;
        const float r = __builtin_amdgcn_rsqf(ms * inv + a.eps);
        const int64_t c0 = 8 * (int64_t)(lane + 64 * k);
        const float4 w0 = *reinterpret_cast<const float4 *>(a.w + c0);
        const float4 w1 = *reinterpret_cast<const float4 *>(a.w + c0 + 4);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (a.bias) {
            const float4 b0 = *reinterpret_cast<const float4 *>(a.bias + c0);
            const float4 b1 = *reinterpret_cast<const float4 *>(a.bias + c0 + 4);
            bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
            bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
        }
        f32x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(v[k][e] * r, wv[e], bv[e]);
        st_bf16x8(a.out + t * a.D + c0, o);
    }
}

}  // namespace

bool block_prologue_supported(int64_t HP, int64_t GN, int64_t H, int64_t W) {
    const int64_t row = 2 * HP + 2 * GN + H;
    return HP % 8 == 0 && GN % 8 == 0 && row % 8 == 0 && W >= 1 && W <= 4;
}

hipError_t launch_block_prologue(const void *zx, const float *conv_w, const float *conv_b, const float *dt_bias,
                                 void *x, void *Bm, void *Cm, float *dt, int64_t B, int64_t L, int64_t H,
                                 int64_t HP, int64_t GN, int64_t W, hipStream_t stream) {
    const int64_t C = HP + 2 * GN;
    const int ctiles = (int)((C / 8 + 255) / 256);
    ProArgs a{(const __bf16 *)zx, conv_w, conv_b, dt_bias, (__bf16 *)x, (__bf16 *)Bm, (__bf16 *)Cm, dt,
              L, HP, GN, H, 2 * HP + 2 * GN + H, ctiles};
    // token tiles run fastest: the hardware deals workgroup i to XCD i mod 8,
    // and with the channel tiles fastest each XCD got one kind of tile only
    // (at the 2.7B shape, 4 kinds: half the XCDs carried the full channel
    // tiles, the others the partial one or the light dt tiles)
    const dim3 grid((unsigned)((L + kTok - 1) / kTok), (unsigned)(ctiles + 1), (unsigned)B);
    switch (W) {
        case 1: prologue_kernel<1><<<grid, 256, 0, stream>>>(a); break;
        case 2: prologue_kernel<2><<<grid, 256, 0, stream>>>(a); break;
        case 3: prologue_kernel<3><<<grid, 256, 0, stream>>>(a); break;
        case 4: prologue_kernel<4><<<grid, 256, 0, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool gated_norm_supported(int64_t D, int64_t ngroups, int64_t zstride) {
    return D % 8 == 0 && D / 8 <= 16 * 64 && ngroups >= 1 && ngroups <= kMaxGroups && D % ngroups == 0 &&
           (D / ngroups) % 8 == 0 && zstride >= D && zstride % 8 == 0;
}

hipError_t launch_gated_norm(const void *y, const void *z, int64_t zstride, const float *w, const float *bias,
                             void *out, int64_t T, int64_t D, int64_t ngroups, float eps, int center,
                             hipStream_t stream) {
    NormArgs a{(const __bf16 *)y, (const __bf16 *)z, w, bias, (__bf16 *)out, T, D, zstride, (int)ngroups,
               center ? 1 : 0, eps};
    const dim3 grid((unsigned)((T + 3) / 4));
    const int kc = (int)((D / 8 + 63) / 64);   // chunks per lane
    switch (kc) {
#define SSD_NORM_CASE(K) \
    case K: gated_norm_kernel<K><<<grid, 256, 0, stream>>>(a); break;
        SSD_NORM_CASE(1) SSD_NORM_CASE(2) SSD_NORM_CASE(3) SSD_NORM_CASE(4) SSD_NORM_CASE(5) SSD_NORM_CASE(6)
        SSD_NORM_CASE(7) SSD_NORM_CASE(8) SSD_NORM_CASE(9) SSD_NORM_CASE(10) SSD_NORM_CASE(11)
        SSD_NORM_CASE(12) SSD_NORM_CASE(13) SSD_NORM_CASE(14) SSD_NORM_CASE(15) SSD_NORM_CASE(16)
#undef SSD_NORM_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
