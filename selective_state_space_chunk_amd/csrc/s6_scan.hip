// Mamba-1 selective scan with diagonal A (the "Mamba" reading notes, section
// 2.2 for the recurrence and the zero-order-hold rule, section 3.2 for the
// input-dependent dt, B, C).  Every channel d and state n is a scalar
// recurrence, h = exp(dt A[d][n]) h + bbar x, y = sum_n C[n] h + D x, so
// the work is vector-ALU arithmetic (one exp2 and a few FMAs per state and
// token), not matrix products.
//
// Workgroup (channel block, b): 64 channels of batch row b, four waves.  Lane
// l of wave w takes channel 16w + l % 16 and its states n = (l / 16) N/4 ..
// + N/4 - 1, so each lane runs N/4 independent chains.  Tokens go in chunks
// of 32: x and dt (32 rows x 128 bytes) are staged in LDS transposed, so
// that a lane reads 8 tokens of its channel at once, and Bm, Cm as they come,
// all from registers loaded one chunk ahead.  A lane keeps its partial sums of
// y for the whole chunk in registers; the four partials of a channel are added
// once per chunk through LDS, and y leaves as whole 128-byte rows.  Tokens
// past the end are zeros (dt = 0, x = 0), which leave the state as it is, so
// every chunk runs all 32 steps unrolled.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssd {

namespace {

struct S6Args {
    const __bf16 *x, *dt, *Bm, *Cm;
    const float *A, *D, *init;
    __bf16 *y;
    float *final_state;
    int64_t L, Dch, G;
    int zoh;
};

constexpr int kCh = 64;   // channels per workgroup
constexpr int kT = 32;    // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;

// kZoh: zero-order-hold input term (else dt Bm x); a template parameter so
// that the unrolled chunk is one block the scheduler can interleave
template <int N, bool kZoh>
__global__ __launch_bounds__(256) void s6_kernel(S6Args a) {
    constexpr int SPL = N / 4;          // states per lane
    constexpr int BCT = kT * N / 8;     // threads that stage Bm (and Cm) of a chunk
    constexpr int XS = kT + 4;          // row of the transposed x / dt tiles (fp32)
    constexpr int YS = kT + 4;          // row of the partial-sum tile (fp32)
    // staged in fp32: the conversions happen once, at staging
    __shared__ __align__(16) float xt[2][kCh][XS];   // [channel][token]
    __shared__ __align__(16) float dtt[2][kCh][XS];
    __shared__ __align__(16) float bs[2][kT][N];
    __shared__ __align__(16) float cs[2][kT][N];
    __shared__ __align__(16) float yq[4][kCh][YS];    // per-quarter partial sums of y
    const int64_t b = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * kCh;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ci = 16 * wave + (lane & 15);
    const int q = lane >> 4;
    const int64_t c = c0 + ci;
    const int64_t g = c0 / (a.Dch / a.G);
    const int64_t L = a.L;

    // zero-order hold: h' = av h + coef Bm x with coef = (av - 1) / A, where
    // A = 0 its limit dt (invA = 0 and zf = 1 there: coef = dt)
    float A2[SPL], invA[SPL], zf[SPL], h[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const int n = q * SPL + j;
        const float Av = a.A[c * N + n];
        A2[j] = Av * kLog2e;
        invA[j] = Av != 0.f ? 1.f / Av : 0.f;
        zf[j] = Av != 0.f ? 0.f : 1.f;
        h[j] = a.init ? a.init[(b * a.Dch + c) * N + n] : 0.f;
    }

    // staging roles: token sr, channels sc .. sc+7 of the x and dt tiles (also
    // the y rows this thread stores); token br, states bcol .. +7 of the Bm and
    // Cm tiles (threads below BCT)
    const int sr = tid >> 3, sc = (tid & 7) * 8;
    const int br = tid / (N / 8), bcol = (tid % (N / 8)) * 8;
    float Dv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) Dv[e] = a.D ? a.D[c0 + sc + e] : 0.f;
    const uint4 zero = {0u, 0u, 0u, 0u};
    uint4 rx, rd, rb = zero, rc = zero;
    auto bf = [](uint32_t w, int hi) { return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16)); };
    auto load = [&](int64_t t0) __attribute__((always_inline)) {
        const int64_t t = t0 + sr;
        const bool ok = t < L;   // tokens past the end read as zeros: dt = 0 and x = 0 leave h as it is
        const int64_t xo = (b * L + (ok ? t : 0)) * a.Dch + c0 + sc;
        rx = ok ? *reinterpret_cast<const uint4 *>(a.x + xo) : zero;
        rd = ok ? *reinterpret_cast<const uint4 *>(a.dt + xo) : zero;
        if (tid < BCT) {
            const int64_t tb = t0 + br;
            const bool okb = tb < L;
            const int64_t bo = ((b * L + (okb ? tb : 0)) * a.G + g) * N + bcol;
            rb = okb ? *reinterpret_cast<const uint4 *>(a.Bm + bo) : zero;
            rc = okb ? *reinterpret_cast<const uint4 *>(a.Cm + bo) : zero;
        }
    };
    auto stage = [&](int buf) __attribute__((always_inline)) {
        const uint32_t wx[4] = {rx.x, rx.y, rx.z, rx.w}, wd[4] = {rd.x, rd.y, rd.z, rd.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            xt[buf][sc + e][sr] = bf(wx[e >> 1], e & 1);
            dtt[buf][sc + e][sr] = bf(wd[e >> 1], e & 1);
        }
        if (tid < BCT) {
            const uint32_t wb[4] = {rb.x, rb.y, rb.z, rb.w}, wc[4] = {rc.x, rc.y, rc.z, rc.w};
            float4 *bo = reinterpret_cast<float4 *>(&bs[buf][br][bcol]);
            float4 *co = reinterpret_cast<float4 *>(&cs[buf][br][bcol]);
            bo[0] = float4{bf(wb[0], 0), bf(wb[0], 1), bf(wb[1], 0), bf(wb[1], 1)};
            bo[1] = float4{bf(wb[2], 0), bf(wb[2], 1), bf(wb[3], 0), bf(wb[3], 1)};
            co[0] = float4{bf(wc[0], 0), bf(wc[0], 1), bf(wc[1], 0), bf(wc[1], 1)};
            co[1] = float4{bf(wc[2], 0), bf(wc[2], 1), bf(wc[3], 0), bf(wc[3], 1)};
        }
    };
    const int nchunks = (int)((L + kT - 1) / kT);
    load(0);
    stage(0);
    if (nchunks > 1) load(kT);
    __syncthreads();
    for (int k = 0; k < nchunks; ++k) {
        const int buf = k & 1;
        const int nt = (int)(L - (int64_t)k * kT < kT ? L - (int64_t)k * kT : kT);
        float yp[kT];
#pragma unroll
        for (int tt = 0; tt < kT; ++tt) {
            const float xv = xt[buf][ci][tt], dv = dtt[buf][ci][tt];
            float bv[SPL], cv[SPL];
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                bv[j] = bs[buf][tt][q * SPL + j];
                cv[j] = cs[buf][tt][q * SPL + j];
            }
            float acc = 0.f;
            if constexpr (kZoh) {
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const float av = __builtin_amdgcn_exp2f(dv * A2[j]);
                    const float coef = __builtin_fmaf(zf[j], dv, __builtin_fmaf(av, invA[j], -invA[j]));
                    h[j] = __builtin_fmaf(av, h[j], coef * (bv[j] * xv));
                    acc = __builtin_fmaf(cv[j], h[j], acc);
                }
            } else {
                const float dtx = dv * xv;
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const float av = __builtin_amdgcn_exp2f(dv * A2[j]);
                    h[j] = __builtin_fmaf(av, h[j], dtx * bv[j]);
                    acc = __builtin_fmaf(cv[j], h[j], acc);
                }
            }
            yp[tt] = acc;
        }
#pragma unroll
        for (int r = 0; r < kT / 4; ++r)
            *reinterpret_cast<float4 *>(&yq[q][ci][4 * r]) = float4{yp[4 * r], yp[4 * r + 1], yp[4 * r + 2], yp[4 * r + 3]};
        __syncthreads();
        // y of token sr, channels sc .. sc+7: the four quarters' partial sums plus D x
        if (sr < nt) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = xt[buf][sc + e][sr];
                o[e] = ((yq[0][sc + e][sr] + yq[1][sc + e][sr]) + (yq[2][sc + e][sr] + yq[3][sc + e][sr])) +
                       Dv[e] * xv;
            }
            typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
            bf16x8_t ov;
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[e] = (__bf16)o[e];
            *reinterpret_cast<bf16x8_t *>(a.y + (b * L + (int64_t)k * kT + sr) * a.Dch + c0 + sc) = ov;
        }
        if (k + 1 < nchunks) {
            stage(buf ^ 1);
            if (k + 2 < nchunks) load((int64_t)(k + 2) * kT);
        }
        __syncthreads();
    }
    if (a.final_state) {
#pragma unroll
        for (int j = 0; j < SPL; ++j) a.final_state[(b * a.Dch + c) * N + q * SPL + j] = h[j];
    }
}

// One state per lane, for N = 8 or 16: the lanes of a channel form one
// DPP row (16 lanes) or half-row (8), so y is summed over them with DPP, no
// LDS.  The sums of N tokens are taken together (a transposing reduction:
// log2 N exchange steps that halve the values each lane holds, ending with
// lane n holding token n's sum), about 3 operations per token where a
// separate row sum per token took 4 and a store from one lane (727 against
// 612 us at the Mamba-1 2.8B shape).  A workgroup takes CW = 256 / N
// channels of one batch row, so there are many small workgroups (Dch / CW
// per row): five per compute unit at the Mamba-1 2.8B shape, every SIMD with
// the same load.  x, dt, Bm and Cm of a chunk are staged transposed in fp32
// ([channel or state][token]), so a lane reads four tokens per LDS load.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, true));
}
// p[t], t < N, held by each of the N lanes of a channel: lane n gets the sum
// over those lanes of p[n].  Each step pairs a lane with one that differs in
// the next bit of n (and in the bits below it): the lane keeps the half of its
// values that its bit names, adds the partner's values for that half, and
// sends the other half; after log2 N steps one value is left, for token n.
template <int N>
__device__ __forceinline__ float lanes_transpose_sum(float (&p)[N], int n) {
    if constexpr (N == 16) {
        const bool hi = n & 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float keep = hi ? p[8 + j] : p[j], send = hi ? p[j] : p[8 + j];
            p[j] = keep + dpp_mov<0x140>(send);   // row_mirror: lane 15 - n
        }
    }
    {
        const bool hi = n & 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float keep = hi ? p[4 + j] : p[j], send = hi ? p[j] : p[4 + j];
            p[j] = keep + dpp_mov<0x141>(send);   // row_half_mirror: lane 7 - n of the 8
        }
    }
    {
        const bool hi = n & 2;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float keep = hi ? p[2 + j] : p[j], send = hi ? p[j] : p[2 + j];
            p[j] = keep + dpp_mov<0x1B>(send);    // quad_perm [3,2,1,0]
        }
    }
    const bool hi = n & 1;
    const float keep = hi ? p[1] : p[0], send = hi ? p[0] : p[1];
    return keep + dpp_mov<0xB1>(send);            // quad_perm [1,0,3,2]
}

// At most 96 registers at N = 16 and 128 at N = 8 (five and four waves per
// SIMD): at N = 16 the five workgroups a compute unit gets at the Mamba-1
// 2.8B shape then run at once.
template <int N, bool kZoh>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(N == 16 ? 5 : 4))) void s6_lane_kernel(S6Args a) {
    constexpr int CW = 256 / N;          // channels per workgroup
    constexpr int TS = kT + 4;           // row of the transposed tiles (fp32)
    constexpr int XU = kT * CW / 8;      // 16-byte units of the x (and dt) tile
    constexpr int BU = kT * N / 8;       // 16-byte units of the Bm (and Cm) tile
    constexpr int UN = 2 * XU + 2 * BU;  // units per chunk
    constexpr int UPT = (UN + 255) / 256;
    __shared__ __align__(16) float xt[2][CW][TS];
    __shared__ __align__(16) float dtt[2][CW][TS];
    __shared__ __align__(16) float bt[2][N][TS];
    __shared__ __align__(16) float ct[2][N][TS];
    __shared__ __align__(16) float yt[kT][CW];
    // D of the workgroup's channels, read from LDS where y leaves (in
    // registers it would spill past the five-wave cap; read from global
    // memory in every chunk it put a load's latency on each chunk: 514
    // against 477 us at the Mamba-1 2.8B shape)
    __shared__ float dsh[CW];
    const int64_t b = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * CW;
    const int tid = threadIdx.x;
    const int ci = tid / N, n = tid % N;
    const int64_t c = c0 + ci;
    const int64_t g = c0 / (a.Dch / a.G);
    const int64_t L = a.L;

    const float Av = a.A[c * N + n];
    const float A2 = Av * kLog2e, invA = Av != 0.f ? 1.f / Av : 0.f, zf = Av != 0.f ? 0.f : 1.f;
    float h = a.init ? a.init[(b * a.Dch + c) * N + n] : 0.f;

    const uint4 zero = {0u, 0u, 0u, 0u};
    uint4 reg[UPT];
    // unit u: x (u < XU), dt, Bm, Cm; row (token) and 8 columns within the tile
    auto unit_src = [&](int u, int64_t t0, const __bf16 *&src, int64_t &off, bool &ok) __attribute__((always_inline)) {
        int k = u, cols = CW;
        const __bf16 *base = a.x;
        if (k >= XU) { k -= XU; base = a.dt; }
        if (u >= 2 * XU) { k = u - 2 * XU; cols = N; base = a.Bm; }
        if (u >= 2 * XU + BU) { k = u - 2 * XU - BU; base = a.Cm; }
        const int per = cols / 8;
        const int r = k / per, col = (k % per) * 8;
        const int64_t t = t0 + r;
        ok = t < L;
        const int64_t tt = ok ? t : 0;
        off = u < 2 * XU ? (b * L + tt) * a.Dch + c0 + col : ((b * L + tt) * a.G + g) * N + col;
        src = base;
    };
    auto load = [&](int64_t t0) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < UPT; ++m) {
            const int u = tid + 256 * m;
            reg[m] = zero;
            if (u < UN) {
                const __bf16 *src;
                int64_t off;
                bool ok;
                unit_src(u, t0, src, off, ok);
                if (ok) reg[m] = *reinterpret_cast<const uint4 *>(src + off);
            }
        }
    };
    auto bf = [](uint32_t w, int hi) { return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16)); };
    auto stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < UPT; ++m) {
            const int u = tid + 256 * m;
            if (u >= UN) continue;
            int k = u, cols = CW;
            float (*dst)[TS] = xt[buf];
            if (u >= XU) { k = u - XU; dst = dtt[buf]; }
            if (u >= 2 * XU) { k = u - 2 * XU; cols = N; dst = bt[buf]; }
            if (u >= 2 * XU + BU) { k = u - 2 * XU - BU; dst = ct[buf]; }
            const int per = cols / 8;
            const int r = k / per, col = (k % per) * 8;
            const uint32_t wv[4] = {reg[m].x, reg[m].y, reg[m].z, reg[m].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[col + e][r] = bf(wv[e >> 1], e & 1);
        }
    };

    const int nchunks = (int)((L + kT - 1) / kT);
    load(0);
    stage(0);
    if (nchunks > 1) load(kT);
    if (tid < CW) dsh[tid] = a.D ? a.D[c0 + tid] : 0.f;
    const bool any_zero = __syncthreads_or(kZoh && Av == 0.f);
    // a state with A = 0 anywhere in the workgroup needs the limit term of the
    // zero-order hold; without one the update is one operation shorter.  The
    // choice is uniform over the workgroup, so each copy of the unrolled chunk
    // loop runs with no branch inside.
    auto chunks = [&](auto limit) __attribute__((always_inline)) {
        constexpr bool kLimit = decltype(limit)::value;
        for (int k = 0; k < nchunks; ++k) {
            const int buf = k & 1;
            const int nt = (int)(L - (int64_t)k * kT < kT ? L - (int64_t)k * kT : kT);
#pragma unroll
            for (int tg = 0; tg < kT; tg += N) {
                float p[N];   // C h of tokens tg .. tg + N - 1 for this lane's state
#pragma unroll
                for (int t4 = 0; t4 < N; t4 += 4) {
                    const float4 x4 = *reinterpret_cast<const float4 *>(&xt[buf][ci][tg + t4]);
                    const float4 d4 = *reinterpret_cast<const float4 *>(&dtt[buf][ci][tg + t4]);
                    const float4 b4 = *reinterpret_cast<const float4 *>(&bt[buf][n][tg + t4]);
                    const float4 c4 = *reinterpret_cast<const float4 *>(&ct[buf][n][tg + t4]);
                    const float xs[4] = {x4.x, x4.y, x4.z, x4.w}, ds[4] = {d4.x, d4.y, d4.z, d4.w};
                    const float bs[4] = {b4.x, b4.y, b4.z, b4.w}, cs[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float av = __builtin_amdgcn_exp2f(ds[e] * A2);
                        if constexpr (kZoh && kLimit) {
                            const float coef = __builtin_fmaf(zf, ds[e], __builtin_fmaf(av, invA, -invA));
                            h = __builtin_fmaf(av, h, coef * (bs[e] * xs[e]));
                        } else if constexpr (kZoh) {
                            // (av - 1) / A Bm x as (av - 1) g, g = Bm x / A, in one rounding
                            const float gx = (invA * bs[e]) * xs[e];
                            h = __builtin_fmaf(av, h, __builtin_fmaf(av, gx, -gx));
                        } else {
                            h = __builtin_fmaf(av, h, (ds[e] * xs[e]) * bs[e]);
                        }
                        p[t4 + e] = cs[e] * h;
                    }
                }
                yt[tg + n][ci] = lanes_transpose_sum<N>(p, n);
            }
            __syncthreads();
            // y rows of the chunk: CW channels (plus D x) per token, 16 bytes per thread
            for (int u = tid; u < kT * CW / 8; u += 256) {
                const int r = u / (CW / 8), col = (u % (CW / 8)) * 8;
                if (r < nt) {
                    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
                    bf16x8_t ov;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        ov[e] = (__bf16)__builtin_fmaf(dsh[col + e], xt[buf][col + e][r], yt[r][col + e]);
                    }
                    *reinterpret_cast<bf16x8_t *>(a.y + (b * L + (int64_t)k * kT + r) * a.Dch + c0 + col) = ov;
                }
            }
            if (k + 1 < nchunks) {
                stage(buf ^ 1);
                if (k + 2 < nchunks) load((int64_t)(k + 2) * kT);
            }
            __syncthreads();
        }
    };
    if (any_zero)
        chunks(std::true_type{});
    else
        chunks(std::false_type{});
    if (a.final_state) a.final_state[(b * a.Dch + c) * N + n] = h;
}

}  // namespace

bool s6_supported(int64_t Dch, int64_t G, int64_t N) {
    return (N == 8 || N == 16 || N == 32) && G >= 1 && Dch % G == 0 && (Dch / G) % kCh == 0;
}

hipError_t launch_s6(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                     const float *init, void *y, float *final_state, int64_t B, int64_t L, int64_t Dch, int64_t G,
                     int64_t N, int zoh, hipStream_t stream) {
    S6Args a{(const __bf16 *)x, (const __bf16 *)dt, (const __bf16 *)Bm, (const __bf16 *)Cm, A, D, init,
             (__bf16 *)y, final_state, L, Dch, G, zoh ? 1 : 0};
    const dim3 grid((unsigned)(Dch / kCh), (unsigned)B);
    // N = 8, 16: one state per lane, 256 / N channels per workgroup
    const dim3 lgrid8((unsigned)(Dch / 32), (unsigned)B), lgrid16((unsigned)(Dch / 16), (unsigned)B);
    switch (N * 2 + (zoh ? 1 : 0)) {
        case 16: s6_lane_kernel<8, false><<<lgrid8, 256, 0, stream>>>(a); break;
        case 17: s6_lane_kernel<8, true><<<lgrid8, 256, 0, stream>>>(a); break;
        case 32: s6_lane_kernel<16, false><<<lgrid16, 256, 0, stream>>>(a); break;
        case 33: s6_lane_kernel<16, true><<<lgrid16, 256, 0, stream>>>(a); break;
        case 64: s6_kernel<32, false><<<grid, 256, 0, stream>>>(a); break;
        case 65: s6_kernel<32, true><<<grid, 256, 0, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
