// Device helpers shared by the libssd kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace ssd {

typedef __bf16 bf16;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float -> bfloat16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Bit pattern of a bfloat16 widened to float.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Inclusive prefix sum of dt*A over a block's first q tokens into lam[0..q),
// and the step sizes into dts[0..q); the rest of lam/dts up to `pad` is filled
// with the last sum and 0 (padding tokens are exact no-ops: dt = 0).  The
// first wave scans 64 values at a time with shuffles, carrying the total from
// one group of 64 to the next.  Every thread of the block must call this.
__device__ inline void block_prefix(const float *dt, int64_t stride, int q, int pad, float Ah,
                                    float *lam, float *dts) {
    if (threadIdx.x < 64) {
        float carry = 0.f;
        for (int base = 0; base < pad; base += 64) {
            const int j = base + (int)threadIdx.x;
            const float d = j < q ? dt[(int64_t)j * stride] : 0.f;
            float v = d * Ah;
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(v, off);
                if ((int)threadIdx.x >= off) v += o;
            }
            v += carry;
            if (j < pad) { lam[j] = v; dts[j] = d; }
            carry = __shfl(v, 63);
        }
    }
    __syncthreads();
}

}  // namespace ssd

// Launchers implemented by the kernel translation units (host side).
namespace ssd {

struct ScanArgs {
    const void *x;
    const float *dt;
    const float *A;
    const void *Bm;
    const void *Cm;
    const float *D;
    const float *init;   // nullable
    void *y;
    float *final_state;  // nullable
    int64_t B, L, H, P, G, N, Q;
    int bf16;            // 1: x, Bm, Cm, y are bfloat16
    hipStream_t stream;
    int varlen = 0;      // 1: dt carries reset flags in its sign bit (packed rows)
};

// Workspace carve-up shared by host code and kernels (regions a call's
// algorithm does not use are not reserved; their pointers are then unusable).
struct Workspace {
    float *states;      // [B, nc, H, P, N]    block states / states entering each block
    float *decay;       // [B, H, nc]          exp(sum of dt*A over the block)
    float *seg;         // segment states of the per-sequence scan and their log2 decays
    size_t seg_floats;  // floats in seg
    void *gram;         // [B*G, blocks, 64, 64] bf16 Cm.Bm^T of every 64-token sub-block
};

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device (the attribute is held per device).  `done` is the call site's
// own record of the devices already set.
constexpr int kMaxDevices = 64;
inline hipError_t allow_lds(const void *kern, size_t bytes, std::atomic<bool> (&done)[kMaxDevices]) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
    // threads that race here all set the same attribute
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done[dev].store(true, std::memory_order_release);
    return e;
}

hipError_t launch_reference_scan(const ScanArgs &a, const Workspace &ws);
// Cm.Bm^T of every 64-token block (matrix-core paths), into ws.gram.
hipError_t launch_gram(const ScanArgs &a, const Workspace &ws, int64_t nsb);
// H_{c+1} = decay_c H_c + S_c over the blocks of every (b, h), in place (the
// state entering each block replaces the block's own state); final state out.
hipError_t launch_state_pass(float *states, const float *decay, const float *init, float *final_state,
                             int64_t B, int64_t H, int64_t PN, int nc, hipStream_t stream);
hipError_t launch_step(float *state, const void *x, const float *dt, const float *A,
                       const void *Bm, const void *Cm, const float *D, void *y,
                       int64_t B, int64_t H, int64_t P, int64_t G, int64_t N, int bf16,
                       hipStream_t stream);

}  // namespace ssd
