// state_update.hip -- one decode token of the selective SSM, state in place.
//
// What it computes (Mamba "Architecture Details" page, "Hardware-Aware
// Implementation / Parallel Algorithm", sequential mode; transition, skip and
// gate as in the scan): for every (b, d),
//     state[b,d,n] <- exp(delta*A[d,n]) * state[b,d,n] + delta*u*B[b,n]
//     y[b,d]        = (sum_n C[b,n]*state[b,d,n] + D[d]*u) * silu(z)
// with y read from the updated state.
//
// Design: pure HBM streaming -- the state is read and written once (it is
// 93% of the bytes at the Mamba-2.8B decode shape).  Four lanes share a
// channel, each owning NS consecutive states, so one wave moves a contiguous
// 64*NS*4-byte stretch of the state with 16-byte vector accesses.  The four
// partial outputs are summed with two cross-lane shuffles (DPP quad
// permutes on gfx950) and lane 0 of the quad writes y.  B and C are shared
// by all channels of a batch row and stay in L2.
#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerChannel = 4;

template <typename T, int NS>
__global__ __launch_bounds__(kThreads) void state_update_kernel(SUParams p) {
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t ch = gid / kLanesPerChannel;        // flattened (b, d)
    const int q = (int)(gid % kLanesPerChannel);      // lane in the quad
    const int64_t nch = p.batch * p.dim;
    const bool cval = ch < nch;
    const int64_t cc = cval ? ch : 0;
    const int64_t b = cc / p.dim, d = cc % p.dim;
    const int N = p.N;
    const int n0 = q * NS;

    const float dl = cval ? Elem<T>::load1(static_cast<const T*>(p.delta) + cc) : 0.f;
    const float u = cval ? Elem<T>::load1(static_cast<const T*>(p.u) + cc) : 0.f;
    const float du = dl * u;

    float h[NS], a[NS], bv[NS], cv[NS];
    float* st = p.state + cc * N + n0;
    const float* Ad = p.A + d * N + n0;
    const T* Bb = static_cast<const T*>(p.Bm) + b * N + n0;
    const T* Cb = static_cast<const T*>(p.Cm) + b * N + n0;
    const bool full = cval && (N == kLanesPerChannel * NS) && (NS % 4 == 0);
    if (full) {
#pragma unroll
        for (int s = 0; s < NS; s += 4) {
            const float4 x = *reinterpret_cast<const float4*>(st + s);
            const float4 y = *reinterpret_cast<const float4*>(Ad + s);
            h[s] = x.x; h[s + 1] = x.y; h[s + 2] = x.z; h[s + 3] = x.w;
            a[s] = y.x; a[s + 1] = y.y; a[s + 2] = y.z; a[s + 3] = y.w;
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            bv[s] = Elem<T>::load1(Bb + s);
            cv[s] = Elem<T>::load1(Cb + s);
        }
    } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bool ok = cval && (n0 + s) < N;
            h[s] = ok ? st[s] : 0.f;
            a[s] = ok ? Ad[s] : 0.f;
            bv[s] = ok ? Elem<T>::load1(Bb + s) : 0.f;
            cv[s] = ok ? Elem<T>::load1(Cb + s) : 0.f;
        }
    }

    float yp = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const float dA = fast_exp2(dl * (a[s] * kLog2e));
        h[s] = fmaf(dA, h[s], du * bv[s]);
        yp = fmaf(cv[s], h[s], yp);
    }

    if (full) {
#pragma unroll
        for (int s = 0; s < NS; s += 4)
            *reinterpret_cast<float4*>(st + s) = make_float4(h[s], h[s + 1], h[s + 2], h[s + 3]);
    } else {
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (cval && (n0 + s) < N) st[s] = h[s];
    }

    // Sum the quad's partial outputs (lanes 4k..4k+3 hold one channel).
    yp += __shfl_xor(yp, 1, kLanesPerChannel);
    yp += __shfl_xor(yp, 2, kLanesPerChannel);
    if (cval && q == 0) {
        float o = yp;
        if (p.Dskip) o = fmaf(p.Dskip[d], u, o);
        if (p.z) o *= silu(Elem<T>::load1(static_cast<const T*>(p.z) + cc));
        Elem<T>::store1(static_cast<T*>(p.y) + cc, o);
    }
}

template <typename T, int NS>
hipError_t launch_ns(const SUParams& p, hipStream_t stream) {
    const int64_t threads = p.batch * p.dim * kLanesPerChannel;
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((state_update_kernel<T, NS>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const SUParams& p, hipStream_t stream) {
    if (p.N <= 4) return launch_ns<T, 1>(p, stream);
    if (p.N <= 8) return launch_ns<T, 2>(p, stream);
    if (p.N <= 16) return launch_ns<T, 4>(p, stream);
    if (p.N <= 32) return launch_ns<T, 8>(p, stream);
    return launch_ns<T, 16>(p, stream);
}

}  // namespace

hipError_t launch_state_update(const SUParams& p, bool is_bf16, hipStream_t stream) {
    return is_bf16 ? launch_t<uint16_t>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace mssm
