// ssd_state_update.hip -- one Mamba-2 decode token, state in place, gfx950.
//
// What it computes ("Mamba - Selective State Space Models" page, "Workflow
// 3": the Mamba-2 block with headdim and d_state; "State-Space Model
// Optimization Patterns" page, section 2: a scalar transition per head): for
// batch row b, head h (group g = h / (H/G)) and head channel p,
//     H[n] <- exp(dt[b,h] * A[h]) * H[n] + dt[b,h] * x[b,h,p] * B[b,g,n]
//     y[b,h,p] = (sum_n C[b,g,n] * H[n] + D[h] * x[b,h,p]) * silu(z[b,h,p])
// with y read from the updated state -- one token of the SSD recurrence.
//
// Design: HBM streaming of the fp32 state [B, H, P, N] (over 99% of the
// bytes at the Mamba-2 decode shape).  LPR lanes share one (b, h, p) row of
// N states; lane l owns the float4s at n = 4 l + 4 LPR v (v < NV), so each
// wave instruction moves whole contiguous rows.  Each thread walks RPT rows
// and issues all of their loads before any arithmetic.  The transition
// exp(dt A) is one value per (b, h), so each row needs one exp.  The row's
// partial outputs are summed with log2(LPR) shuffles and the row's first
// lane writes y.  Loads use clamped indices and are unconditional; stores
// are predicated.  The state is streamed with non-temporal loads and stores.
// d_state 16, 32, 64, 128 and 256 take that kernel; every other d_state up to
// 256 a plain one with element loads.
#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kThreads = 256;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Four consecutive elements of type T at p (aligned to 4 * sizeof(T)), widened.
template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]) {
    if constexpr (sizeof(T) == 4) {
        const float4 x = *reinterpret_cast<const float4*>(p);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xffff0000u);
        v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xffff0000u);
    }
}

template <typename T, int LPR, int NV, int RPT>
__global__ __launch_bounds__(kThreads) void ssd_state_update_kernel(SSDUParams p) {
    constexpr int N = 4 * NV * LPR;
    constexpr int SLOTS = kThreads / LPR;        // rows per block per pass
    const int l = threadIdx.x % LPR;
    const int slot = threadIdx.x / LPR;
    const int64_t nrows = p.batch * p.H * p.P;
    const int hpg = p.H / p.G;

    int64_t row[RPT];
    bool ok[RPT];
    float h[RPT][NV][4], bv[RPT][NV][4], cv[RPT][NV][4];
    float xv[RPT], dtv[RPT], zv[RPT], av[RPT], dsk[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int64_t r = ((int64_t)blockIdx.x * RPT + j) * SLOTS + slot;
        ok[j] = r < nrows;
        row[j] = ok[j] ? r : nrows - 1;
        const int64_t bh = row[j] / p.P;
        const int hh = (int)(bh % p.H);
        const int64_t b = bh / p.H;
        const int64_t bg = b * p.G + hh / hpg;
        const float* st = p.state + row[j] * N + 4 * l;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const f32x4_t s4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(st + 4 * LPR * v));
            h[j][v][0] = s4[0]; h[j][v][1] = s4[1]; h[j][v][2] = s4[2]; h[j][v][3] = s4[3];
            load4(static_cast<const T*>(p.Bm) + bg * N + 4 * l + 4 * LPR * v, bv[j][v]);
            load4(static_cast<const T*>(p.Cm) + bg * N + 4 * l + 4 * LPR * v, cv[j][v]);
        }
        xv[j] = Elem<T>::load1(static_cast<const T*>(p.x) + row[j]);
        dtv[j] = Elem<T>::load1(static_cast<const T*>(p.dt) + bh);
        zv[j] = p.z ? Elem<T>::load1(static_cast<const T*>(p.z) + row[j]) : 0.f;
        av[j] = p.A[hh];
        dsk[j] = p.Dskip ? p.Dskip[hh] : 0.f;
    }

#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const float dA = fast_exp2(dtv[j] * (av[j] * kLog2e));
        const float dx = dtv[j] * xv[j];
        float yp = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[j][v][e] = fmaf(dA, h[j][v][e], dx * bv[j][v][e]);
                yp = fmaf(cv[j][v][e], h[j][v][e], yp);
            }
        if (ok[j]) {
            float* st = p.state + row[j] * N + 4 * l;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                __builtin_nontemporal_store(f32x4_t{h[j][v][0], h[j][v][1], h[j][v][2], h[j][v][3]},
                                            reinterpret_cast<f32x4_t*>(st + 4 * LPR * v));
        }
#pragma unroll
        for (int d = 1; d < LPR; d <<= 1) yp += __shfl_xor(yp, d, LPR);
        if (ok[j] && l == 0) {
            float o = fmaf(dsk[j], xv[j], yp);
            if (p.z) o *= silu(zv[j]);
            Elem<T>::store1(static_cast<T*>(p.y) + row[j], o);
        }
    }
}

// Any d_state up to 256 (the sizes the kernel above does not take): 16 lanes
// per (b, h, p) row, lane l owning states l, l + 16, ...; element loads at
// clamped indices, the states past d_state masked out.  One row per 16 lanes,
// 16 rows per block.
template <typename T>
__global__ __launch_bounds__(kThreads) void ssd_state_update_any_kernel(SSDUParams p) {
    constexpr int LPR = 16, MAXI = 256 / LPR;
    const int l = threadIdx.x % LPR;
    const int64_t nrows = p.batch * p.H * p.P;
    const int64_t r = (int64_t)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR;
    const bool ok = r < nrows;
    const int64_t row = ok ? r : nrows - 1;
    const int64_t bh = row / p.P;
    const int hh = (int)(bh % p.H);
    const int64_t bg = (bh / p.H) * p.G + hh / (p.H / p.G);
    const int N = p.N;
    const float xv = Elem<T>::load1(static_cast<const T*>(p.x) + row);
    const float dtv = Elem<T>::load1(static_cast<const T*>(p.dt) + bh);
    const float zv = p.z ? Elem<T>::load1(static_cast<const T*>(p.z) + row) : 0.f;
    const float dA = fast_exp2(dtv * (p.A[hh] * kLog2e));
    const float dx = dtv * xv;
    float* st = p.state + row * N;
    const T* Bb = static_cast<const T*>(p.Bm) + bg * N;
    const T* Cb = static_cast<const T*>(p.Cm) + bg * N;
    float yp = 0.f;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        if (LPR * i >= N) break;                 // the same for every lane
        const int n = l + LPR * i;
        const bool nv = n < N;
        const int nn = nv ? n : N - 1;
        const float hv = fmaf(dA, st[nn], dx * Elem<T>::load1(Bb + nn));
        if (nv) {
            yp = fmaf(Elem<T>::load1(Cb + nn), hv, yp);
            if (ok) st[n] = hv;
        }
    }
#pragma unroll
    for (int d = 1; d < LPR; d <<= 1) yp += __shfl_xor(yp, d, LPR);
    if (ok && l == 0) {
        float o = fmaf(p.Dskip ? p.Dskip[hh] : 0.f, xv, yp);
        if (p.z) o *= silu(zv);
        Elem<T>::store1(static_cast<T*>(p.y) + row, o);
    }
}

template <typename T, int LPR, int NV>
hipError_t launch_cfg(const SSDUParams& p, hipStream_t stream) {
    constexpr int RPT = 2;
    constexpr int rows_per_block = (kThreads / LPR) * RPT;
    const int64_t nrows = p.batch * p.H * p.P;
    const int64_t blocks = (nrows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((ssd_state_update_kernel<T, LPR, NV, RPT>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const SSDUParams& p, hipStream_t stream) {
    switch (p.N) {
        case 16: return launch_cfg<T, 4, 1>(p, stream);
        case 32: return launch_cfg<T, 8, 1>(p, stream);
        case 64: return launch_cfg<T, 16, 1>(p, stream);
        case 128: return launch_cfg<T, 32, 1>(p, stream);
        case 256: return launch_cfg<T, 32, 2>(p, stream);
        default: {
            if (p.N < 1 || p.N > 256) return hipErrorInvalidValue;
            const int64_t blocks = (p.batch * p.H * p.P + 15) / 16;
            if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((ssd_state_update_any_kernel<T>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
            return hipGetLastError();
        }
    }
}

}  // namespace

bool ssd_state_update_supported(int64_t N) { return N >= 1 && N <= 256; }

hipError_t launch_ssd_state_update(const SSDUParams& p, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? launch_t<uint16_t>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace mssm
