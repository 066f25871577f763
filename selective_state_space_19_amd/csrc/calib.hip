// calib.hip -- measurement kernels for the benchmark (libmssm_calib.so).
//
// Not part of the scan library: these kernels give the benchmark the
// ceilings its roofline figures are read against, measured on the GPU at
// hand.
//   * stream copy:  dst[i] = src[i], 16-byte vectors, grid-stride -- the
//     streaming-copy ceiling of HBM (bytes read + bytes written per second);
//   * stream read:  a sum over src, 16-byte vectors -- the read-only ceiling
//     (the S6 scan reads three bytes for every one it writes);
//   * VALU issue probes: every lane runs independent chains of one
//     instruction kind for a fixed count, so the elapsed time gives the
//     issue rate in lane-instructions per second:
//       mode 0  v_fma_f32 chains;
//       mode 1  v_exp_f32 chains;
//       mode 2  the S6 scan's work per state element -- v_mul (step times
//               A), v_exp_f32, v_mul (step*u times B), v_fma (state),
//               v_fma (output) -- laid out as the scan kernel runs a group:
//               16 tokens x 2 states per lane, the decay factors and input
//               terms of the group first, then the recurrence, the per-token
//               (step, step*u) pairs read from LDS; the time per element is
//               the scan's arithmetic floor on this chip;
//       mode 3  16 v_exp_f32 and 64 independent v_fma_f32 per iteration:
//               whether the exponentials overlap the FMAs (time near the
//               larger of the two) or add to them (near the sum);
//       mode 7  mode 2 with B and C read from memory as wave-uniform values
//               (scalar registers), as the scan kernel takes them.
// The grid sets the occupancy: 2048 workgroups of 256 threads are 8 waves
// per SIMD, 512 are the 2 scan waves per SIMD of the S6 kernel.
// Entry points are extern "C" with plain pointers; they return hipError_t
// values as int.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        __builtin_nontemporal_store(v, dst + i);
    }
}

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ out,
                                                          int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // one store per thread keeps the loads live; `out` has a slot per thread
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

constexpr int kChains = 16;

__global__ __launch_bounds__(256) void valu_probe_kernel(float* __restrict__ out, const float* __restrict__ uni,
                                                         int iters, int mode, float seed) {
    const int tid = blockIdx.x * blockDim.x + threadIdx.x;
    __shared__ float4 s_dd[8][256];               // per-token (step, step*u) pairs of one group, per lane
    if (mode == 2 || mode == 7) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            s_dd[k][threadIdx.x] = make_float4(0.01f * (k + 1), 0.02f, 0.011f * (k + 1), 0.03f + seed);
        __syncthreads();
        const float a2[2] = {-1.4426950f * (1.f + (threadIdx.x & 1)), -2.8853900f};
        float bB[2] = {0.7f + 1e-3f * (threadIdx.x & 3), -0.3f}, cC[2] = {0.2f, 0.9f + 1e-3f * (threadIdx.x & 7)};
        if (mode == 7) {                          // wave-uniform: scalar loads into scalar registers
            bB[0] = uni[1]; bB[1] = uni[2]; cC[0] = uni[3]; cC[1] = uni[4];
        }
        float h[2] = {seed, -seed};
        float yv[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < iters; ++i) {
            float dA[16][2], bu[16][2];
#pragma unroll
            for (int k = 0; k < 16; k += 2) {
                const float4 q = s_dd[k / 2][threadIdx.x];
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    dA[k][st] = __builtin_amdgcn_exp2f(q.x * a2[st]);
                    dA[k + 1][st] = __builtin_amdgcn_exp2f(q.z * a2[st]);
                    bu[k][st] = q.y * bB[st];
                    bu[k + 1][st] = q.w * bB[st];
                }
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    h[st] = fmaf(dA[k][st], h[st], bu[k][st]);
                    yv[k & 3] = fmaf(cC[st], h[st], yv[k & 3]);
                }
            asm volatile("" ::: "memory");        // the LDS pairs are re-read every group, as in the scan
        }
        out[tid] = h[0] + h[1] + yv[0] + yv[1] + yv[2] + yv[3];
        return;
    }
    if (mode == 3) {
        float e[16], f[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            e[k] = seed * (float)(k + 1);
            f[k] = seed + (float)k;
        }
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                e[k] = __builtin_amdgcn_exp2f(-__builtin_fabsf(e[k]));
#pragma unroll
                for (int r = 0; r < 4; ++r) f[(k + 5 * r) & 15] = fmaf(f[(k + 5 * r) & 15], 0.999f, 1e-3f);
            }
        }
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) sum += e[k] + f[k];
        out[tid] = sum;
        return;
    }
    float v[kChains], a[kChains], c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
        v[k] = seed * (float)(k + 1) + 1e-3f * (float)(threadIdx.x & 63);
        a[k] = -0.0625f * (float)(k + 1);
        c[k] = 0.5f + 0.01f * (float)k;
    }
    if (mode == 0) {
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < kChains; ++k) v[k] = fmaf(v[k], c[k], a[k]);
        }
    } else if (mode == 1) {
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < kChains; ++k) v[k] = __builtin_amdgcn_exp2f(-__builtin_fabsf(v[k]));
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += v[k];
    out[tid] = s;
}

}  // namespace

extern "C" {

// dst <- src, n_bytes a multiple of 16, both 16-byte aligned.
int mssm_calib_copy(const void* src, void* dst, int64_t n_bytes, int blocks, void* stream) {
    hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n_bytes / 16);
    return (int)hipGetLastError();
}

// Reads n_bytes of src; out holds blocks * 256 uint32 slots.
int mssm_calib_read(const void* src, uint32_t* out, int64_t n_bytes, int blocks, void* stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src), out, n_bytes / 16);
    return (int)hipGetLastError();
}

// out holds blocks * 256 floats; uni holds 8 wave-uniform inputs.  Per lane
// and iteration: 16 instructions of the probed kind (modes 0, 1); 32 scan
// elements (modes 2, 7); 16 exponentials and 64 FMAs (mode 3).
int mssm_calib_valu(float* out, const float* uni, int blocks, int iters, int mode, float seed, void* stream) {
    hipLaunchKernelGGL(valu_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, uni, iters, mode,
                       seed);
    return (int)hipGetLastError();
}

}  // extern "C"
