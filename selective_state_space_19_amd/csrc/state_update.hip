// state_update.hip -- one decode token of the selective SSM, state in place.
//
// What it computes ("Mamba Architecture Details" page, "Hardware-Aware
// Implementation / Parallel Algorithm", sequential mode; transition, skip and
// gate as in the scan): for every (b, d),
//     state[b,d,n] <- exp(delta*A[d,n]) * state[b,d,n] + delta*u*B[b,n]
//     y[b,d]        = (sum_n C[b,n]*state[b,d,n] + D[d]*u) * silu(z)
// with y read from the updated state.
//
// Design: pure HBM streaming -- the state is read and written once (it is
// 93% of the bytes at the Mamba-2.8B decode shape), so the kernel's job is to
// keep enough of it in flight.  Four lanes share a channel, each owning NS
// consecutive states, so one wave instruction moves a contiguous 16-channel
// stretch of the state with 16-byte accesses; each thread handles one
// channel d in RPT batch rows and issues all of their loads before any
// arithmetic (RPT * NS * 4 bytes of state in flight per lane), reading A[d]
// and D[d] once for all RPT rows.  Loads use clamped indices and are
// unconditional; only the stores are predicated.  The quad's partial outputs
// are summed with two cross-lane shuffles and the quad's first lane writes y.
// B and C are per batch row and shared by all channels (they stay in L2).
// The state is loaded and stored non-temporally: each call touches it once,
// and a model cycles through one such state per layer, so caching it only
// evicts the small operands that are reused.
#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerChannel = 4;
constexpr int kQuadsPerBlock = kThreads / kLanesPerChannel;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// NS contiguous elements of type T starting at p, widened to float.  p is
// aligned to NS * sizeof(T) when VEC (then one vector load per 16 bytes).
// STREAM marks data touched once per call (the state): non-temporal loads.
template <typename T, int NS, bool VEC, bool STREAM = false>
__device__ __forceinline__ void load_run(const T* p, int valid, float (&v)[NS]) {
    if constexpr (VEC && sizeof(T) == 4 && NS % 4 == 0) {
#pragma unroll
        for (int s = 0; s < NS; s += 4) {
            const f32x4_t* a = reinterpret_cast<const f32x4_t*>(p + s);
            const f32x4_t x = STREAM ? __builtin_nontemporal_load(a) : *a;
            v[s] = x[0]; v[s + 1] = x[1]; v[s + 2] = x[2]; v[s + 3] = x[3];
        }
    } else if constexpr (VEC && sizeof(T) == 2 && NS % 4 == 0) {
#pragma unroll
        for (int s = 0; s < NS; s += 4) {
            const uint2 x = *reinterpret_cast<const uint2*>(p + s);
            v[s] = __uint_as_float(x.x << 16); v[s + 1] = __uint_as_float(x.x & 0xffff0000u);
            v[s + 2] = __uint_as_float(x.y << 16); v[s + 3] = __uint_as_float(x.y & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float x = Elem<T>::load1(p + (s < valid ? s : 0));   // clamped: always a valid address
            v[s] = s < valid ? x : 0.f;
        }
    }
}

template <typename T, int NS, int RPT, bool VEC>
__global__ __launch_bounds__(kThreads) void state_update_kernel(SUParams p) {
    // Block = 64 consecutive channels d x RPT consecutive batch rows b; a quad
    // owns one d and walks the RPT rows, so A[d] and D[d] are read once.
    const int q = threadIdx.x % kLanesPerChannel;
    const uint32_t nbx = (uint32_t)((p.dim + kQuadsPerBlock - 1) / kQuadsPerBlock);
    const uint32_t bx = blockIdx.x % nbx, by = blockIdx.x / nbx;   // 1-D grid: no per-axis limits
    const int64_t d = (int64_t)bx * kQuadsPerBlock + threadIdx.x / kLanesPerChannel;
    const bool dval = d < p.dim;
    const int64_t dc = dval ? d : p.dim - 1;
    const int N = p.N;
    const int n0 = q * NS;
    const int valid = VEC ? NS : (N - n0 < 0 ? 0 : (N - n0 > NS ? NS : N - n0));
    const int nn0 = VEC ? n0 : (n0 < N ? n0 : 0);     // first state this lane touches (clamped)

    float a[NS];
    load_run<float, NS, VEC>(p.A + dc * N + nn0, valid, a);
#pragma unroll
    for (int s = 0; s < NS; ++s) a[s] *= kLog2e;
    const float dsk = p.Dskip ? p.Dskip[dc] : 0.f;

    int64_t cc[RPT];
    bool ok[RPT];
    float h[RPT][NS], bv[RPT][NS], cv[RPT][NS], dl[RPT], uu[RPT], zz[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int64_t b = (int64_t)by * RPT + j;
        ok[j] = dval && b < p.batch;
        const int64_t bc = b < p.batch ? b : p.batch - 1;
        cc[j] = bc * p.dim + dc;
        load_run<float, NS, VEC, true>(p.state + cc[j] * N + nn0, valid, h[j]);
        load_run<T, NS, VEC>(static_cast<const T*>(p.Bm) + bc * N + nn0, valid, bv[j]);
        load_run<T, NS, VEC>(static_cast<const T*>(p.Cm) + bc * N + nn0, valid, cv[j]);
        dl[j] = Elem<T>::load1(static_cast<const T*>(p.delta) + cc[j]);
        uu[j] = Elem<T>::load1(static_cast<const T*>(p.u) + cc[j]);
        zz[j] = p.z ? Elem<T>::load1(static_cast<const T*>(p.z) + cc[j]) : 0.f;
    }

#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const float du = dl[j] * uu[j];
        float yp = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float dA = fast_exp2(dl[j] * a[s]);
            h[j][s] = fmaf(dA, h[j][s], du * bv[j][s]);
            yp = fmaf(cv[j][s], h[j][s], yp);
        }
        float* st = p.state + cc[j] * N + nn0;
        if (ok[j]) {
            if constexpr (VEC) {
#pragma unroll
                for (int s = 0; s < NS; s += 4)
                    __builtin_nontemporal_store(f32x4_t{h[j][s], h[j][s + 1], h[j][s + 2], h[j][s + 3]},
                                                reinterpret_cast<f32x4_t*>(st + s));
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    if (s < valid) st[s] = h[j][s];
            }
        }
        // Sum the quad's partial outputs (lanes 4k..4k+3 hold one channel).
        yp += __shfl_xor(yp, 1, kLanesPerChannel);
        yp += __shfl_xor(yp, 2, kLanesPerChannel);
        if (ok[j] && q == 0) {
            float o = fmaf(dsk, uu[j], yp);
            if (p.z) o *= silu(zz[j]);
            Elem<T>::store1(static_cast<T*>(p.y) + cc[j], o);
        }
    }
}

template <typename T, int NS, int RPT>
hipError_t launch_ns(const SUParams& p, hipStream_t stream) {
    const int64_t blocks = ((p.dim + kQuadsPerBlock - 1) / kQuadsPerBlock) * ((p.batch + RPT - 1) / RPT);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    if (p.N == kLanesPerChannel * NS && NS % 4 == 0)
        hipLaunchKernelGGL((state_update_kernel<T, NS, RPT, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((state_update_kernel<T, NS, RPT, false>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// Batch rows per thread: about 8-16 states (32-64 bytes) of loads in flight
// per lane.
template <typename T>
hipError_t launch_t(const SUParams& p, hipStream_t stream) {
    if (p.N <= 4) return launch_ns<T, 1, 8>(p, stream);
    if (p.N <= 8) return launch_ns<T, 2, 4>(p, stream);
    if (p.N <= 16) return launch_ns<T, 4, 2>(p, stream);
    if (p.N <= 32) return launch_ns<T, 8, 2>(p, stream);
    return launch_ns<T, 16, 1>(p, stream);
}

}  // namespace

hipError_t launch_state_update(const SUParams& p, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? launch_t<uint16_t>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace mssm
