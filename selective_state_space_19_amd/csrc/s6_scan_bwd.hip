// s6_scan_bwd.hip -- backward of the S6 selective scan for gfx950.
//
// What it computes: the reverse-mode derivative of the scan in s6_scan.hip
// ("State-Space Model Optimization Patterns" page, section 4: the training
// pass recomputes the forward states instead of storing them all; the
// recurrence is that of the "Mamba Architecture Details" page, "Selective
// State Space Mechanism").  For the loss sum(dout * out) + sum(dhT * h_final),
// with g_t = dout_t * silu(z_t), a_t = exp(delta_t A) and the adjoint
// lambda_t = dL/dh_t taken backwards in time:
//     lambda_t = a_{t+1} lambda_{t+1} + g_t C_t      (dhT at the last token)
//     dC_t += g_t h_t,  dB_t += lambda_t delta_t u_t   (summed over channels)
//     du_t = g_t D + sum_n lambda_t delta_t B_t
//     ddelta_t = sum_n lambda_t (A a_t h_{t-1} + u_t B_t)
//     dA += lambda_t delta_t a_t h_{t-1},  dD += g_t u_t
//     dz_t = dout_t y_t silu'(z_t),  dh0 = a_0 lambda_0.
//
// Design: a workgroup of 8 waves owns 64 channels of one batch row; lane =
// channel, wave w = states [w NS, (w+1) NS).  Row threads (8 per channel)
// load u, delta, dout, z and the whole block's B / C rows ahead of use, the
// chunks whose runs share a 128-byte line together (a line group), so their
// memory latency hides behind the current chunk and each line is fetched
// once; B / C reach the waves through LDS (uniform reads).
//   1. Forward sweep over the whole sequence in chunks of TC tokens (16, or 8
//      when a lane holds more than 2 states), writing
//      the state at every chunk start to the workspace (one fp32 per
//      channel, state and chunk).  Left out (SAVED) when the forward scan
//      has already stored those states there.
//   2. Backward sweep, last chunk first: stage (delta, delta*u, u, g) of the
//      chunk in LDS; recompute the chunk's TC states from its checkpoint into
//      registers (the per-wave partial outputs go to LDS, from which the row
//      threads form y and dz); then walk the chunk backwards, keeping lambda
//      in registers.  dB and dC are summed over the wave's 64 channels (a
//      transposing lane reduction that leaves one value per lane) and stored
//      as this workgroup's partial sums; a second kernel adds the partials of
//      all channel blocks (no atomics: dB and dC are deterministic).  du and
//      ddelta are summed over the waves through LDS by the row threads.
//   dA and dD are accumulated in registers and added with atomics at the end
//   (the entry point zeroes them first).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kNW = 8;                 // waves per workgroup
constexpr int kSegs = 8;               // row threads per channel

// Tokens per chunk: the chunk's states are held in registers (TC x NS).
template <int NS> struct ChunkLen { static constexpr int value = NS <= 2 ? 16 : 8; };

// ---- sums over a wave's 64 lanes of many values at once -----------------------
// A transposing reduction: each step takes two registers x, y and leaves one,
// in which the lanes with a given lane bit 0 hold x summed with the partner
// lane's x, and those with the bit 1 hold y summed likewise.  Step ST uses lane
// bit 5 - ST: ST 0 and 1 are the gfx950 lane swaps across halves and rows (no
// selects needed), ST 2..5 pair lanes inside a row of 16 with DPP (rotate by 8,
// half-row mirror, quad permutes ^2 and ^1; any partner with the other bit
// value works).  After all six steps a register's lane L holds the sum over all
// 64 lanes of the value whose index has L as its top six bits.
template <int ST>
__device__ __forceinline__ float combine(float x, float y) {
    if constexpr (ST == 0 || ST == 1) {
        const auto r = ST == 0 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false)
                               : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        constexpr int CTRL = ST == 2 ? 0x128 : ST == 3 ? 0x141 : ST == 4 ? 0x4e : 0xb1;
        const bool hi = (__lane_id() >> (5 - ST)) & 1;
        const float keep = hi ? y : x, send = hi ? x : y;
        // (every lane has a source lane for these patterns; the zero `old`
        // lets the move fold into the add as one DPP instruction)
        return keep + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), CTRL,
                                                                             0xf, 0xf, false));
    }
}

// Steps ST, ST + 1, ... on v[0 .. SIZE) (pairs v[i], v[i + SIZE / 2]) until one
// register is left or the six steps are done.
template <int ST, int SIZE, int CAP>
__device__ __forceinline__ void tree(float (&v)[CAP]) {
    if constexpr (SIZE > 1 && ST < 6) {
#pragma unroll
        for (int i = 0; i < SIZE / 2; ++i) v[i] = combine<ST>(v[i], v[i + SIZE / 2]);
        tree<ST + 1, SIZE / 2>(v);
    }
}

constexpr int log2i(int n) { return n <= 1 ? 0 : 1 + log2i(n / 2); }

// f(integral_constant<int, i>) for i = I, I - 1, .., 0, unrolled at compile time.
template <int I, typename F>
__device__ __forceinline__ void down_for(F&& f) {
    f(std::integral_constant<int, I>{});
    if constexpr (I > 0) down_for<I - 1>(f);
}

// Chunks whose row runs (TC tokens of T) share one 128-byte line, at most 4.
// The row threads load the runs of such a group of chunks together, so every
// line is fetched from HBM once, not once per chunk when L2 has evicted it in
// between.
template <typename T, int TC> constexpr int kLineGroup =
    128 / (TC * int(sizeof(T))) < 1 ? 1 : (128 / (TC * int(sizeof(T))) > 4 ? 4 : 128 / (TC * int(sizeof(T))));

// Values made opaque to the optimiser (an empty asm on each 32-bit word).
__device__ __forceinline__ void opaque(uint32_t& x) { asm("" : "+v"(x)); }
__device__ __forceinline__ void opaque(uint2& x) { asm("" : "+v"(x.x)); asm("" : "+v"(x.y)); }
__device__ __forceinline__ void opaque(float& x) { asm("" : "+v"(x)); }
__device__ __forceinline__ void opaque(uint16_t& x) {
    uint32_t y = x;
    asm("" : "+v"(y));
    x = (uint16_t)y;
}

// a[i] for a wave-uniform i < G, as a chain of selects.  The elements go
// through `opaque` first: a select between two array elements could
// otherwise become one load at a computed index, which would move the whole
// array to scratch memory.
template <int G, typename V>
__device__ __forceinline__ V pick(const V (&a)[G], int i) {
    V v = a[0];
    opaque(v);
#pragma unroll
    for (int k = 1; k < G; ++k) {
        V x = a[k];
        opaque(x);
        v = i == k ? x : v;
    }
    return v;
}

// Element c of a line group's registers: a direct index when c is a
// compile-time constant, else the select chain of `pick`.
template <int G, typename V, int C>
__device__ __forceinline__ V sel(const V (&a)[G], std::integral_constant<int, C>) { return a[C]; }
template <int G, typename V>
__device__ __forceinline__ V sel(const V (&a)[G], int c) { return pick(a, c); }
template <int C> constexpr int index_of(std::integral_constant<int, C>) { return C; }
__device__ __forceinline__ int index_of(int c) { return c; }

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// An element of type T widened to float (bf16: the upper half of a float).
__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// BUF (L even, a block's rows addressable with 32-bit offsets): each row
// thread reads its two tokens with one buffer load per array; offsets past the
// sequence or past the block's rows read zero.  Otherwise element loads.
// SAVED: the workspace already holds the chunk-start states (written by the
// forward scan), so the forward sweep is left out.
template <typename T, int NS, bool BUF, bool SAVED>
__global__ __launch_bounds__(kNW * 64) void s6_scan_bwd_kernel(S6BwdParams p) {
    constexpr int kTC = ChunkLen<NS>::value;
    constexpr int kTPT = kTC / kSegs;      // tokens per row thread
    constexpr int kLG = kLineGroup<T, kTC>;
    __shared__ float4 s_tk[kTC][64 + 1];          // (delta, delta*u, u, g) per token and channel
    __shared__ float s_y[kNW][kTC][64 + 1];       // per-wave partial sum_n C h
    __shared__ float2 s_p[kNW][kTC][64 + 1];      // per-wave partial (du, ddelta)
    __shared__ __align__(16) float s_bc[2][2][kNW * NS][kTC];   // [buffer][B 0 / C 1][state][token]
    __shared__ float2 s_fw[2][kTC][64 + 1];       // forward sweep: (delta, delta*u), double-buffered

    const T* u_in = static_cast<const T*>(p.u);
    const T* dl_in = static_cast<const T*>(p.delta);
    const T* z_in = static_cast<const T*>(p.z);
    const T* go_in = static_cast<const T*>(p.dout);
    const T* __restrict__ B_in = static_cast<const T*>(p.Bm);
    const T* __restrict__ C_in = static_cast<const T*>(p.Cm);
    const int64_t dim = p.dim;
    const int L = p.L, N = p.N;
    const int nck = (L + kTC - 1) / kTC;

    const int tid = threadIdx.x;
    const int64_t nblk_d = (dim + 63) / 64;
    constexpr int kNSP = NS < 2 ? 2 : NS;                 // states per wave in the dB / dC layout
    constexpr int kVPW = 2 * kNSP * kTC;                  // dB / dC partials per wave and chunk
    static_assert(kVPW == 64 || kVPW == 128, "reduction layout");
    const int64_t b = blockIdx.x / nblk_d;
    const int64_t dblk = blockIdx.x % nblk_d;
    const int64_t d0 = dblk * 64;
    const int nrows = (int)((dim - d0) < 64 ? (dim - d0) : 64);

    // ---- scan mapping: lane = channel cs, wave = state group w ----------------
    const int cs = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool cval = cs < nrows;
    const int64_t ch = b * dim + d0 + (cval ? cs : 0);            // (b, d) of this lane
    float a2[NS], Af[NS], h[NS], lam[NS], dAacc[NS];
    int nst[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int n = w * NS + s;
        nst[s] = n < N ? n : 0;
        const bool ok = cval && n < N;
        Af[s] = ok ? p.A[(d0 + cs) * N + n] : 0.f;
        a2[s] = Af[s] * kLog2e;
        h[s] = (ok && p.h0) ? p.h0[ch * N + n] : 0.f;
        lam[s] = (ok && p.dhT) ? p.dhT[ch * N + n] : 0.f;
        dAacc[s] = 0.f;
    }
    // B / C of this wave's states over one chunk (0 past the end or for a
    // state past N), read from LDS after the barrier.  The block's B / C
    // elements of a chunk are fetched by all threads one chunk ahead (raw,
    // clamped addresses; kBPT per thread) and written to s_bc when staging.
    float Bf[NS][kTC], Cf[NS][kTC];
    constexpr int kNP = kNW * NS;                              // states, padded
    constexpr int kBCE = 2 * kNP * kTC;                        // B / C elements per chunk
    constexpr int kBPT = (kBCE + kNW * 64 - 1) / (kNW * 64);   // per thread
    auto bc_index = [&](int i, int& m, int& n, int& k) {
        m = i / (kNP * kTC);
        n = (i / kTC) % kNP;
        k = i % kTC;
    };
    auto fetch_bc = [&](int ck, T (&r)[kBPT]) {
#pragma unroll
        for (int q = 0; q < kBPT; ++q) {
            const int i = tid + q * kNW * 64;
            int m, n, k;
            bc_index(i < kBCE ? i : 0, m, n, k);
            const int t = ck * kTC + k;
            r[q] = (m ? C_in : B_in)[(b * N + (n < N ? n : N - 1)) * (int64_t)L + (t < L ? t : L - 1)];
        }
    };
    auto stage_bc = [&](int ck, const T (&r)[kBPT], int buf) {
#pragma unroll
        for (int q = 0; q < kBPT; ++q) {
            const int i = tid + q * kNW * 64;
            if (i < kBCE) {
                int m, n, k;
                bc_index(i, m, n, k);
                const float v = widen(r[q]);
                s_bc[buf][m][n][k] = (n < N && ck * kTC + k < L) ? v : 0.f;
            }
        }
    };
    auto read_bc = [&](int buf) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int k = 0; k < kTC; k += 4) {
                const float4 x = *reinterpret_cast<const float4*>(&s_bc[buf][0][w * NS + s][k]);
                const float4 y = *reinterpret_cast<const float4*>(&s_bc[buf][1][w * NS + s][k]);
                Bf[s][k] = x.x; Bf[s][k + 1] = x.y; Bf[s][k + 2] = x.z; Bf[s][k + 3] = x.w;
                Cf[s][k] = y.x; Cf[s][k + 1] = y.y; Cf[s][k + 2] = y.z; Cf[s][k + 3] = y.w;
            }
    };
    // checkpoint of state s at the start of chunk ck (a lane or state past the
    // end reads a valid element in place of its own: clamped, never used)
    auto ckpt = [&](int ck, int s) -> float* {
        return p.ws + ((b * nck + ck) * (int64_t)N + w * NS + s) * dim + d0 + cs;
    };
    auto ckpt_in = [&](int ck, int s) -> const float* {
        return p.ws + ((b * nck + ck) * (int64_t)N + nst[s]) * dim + d0 + (cval ? cs : 0);
    };

    // ---- row mapping: thread -> (row cr, tokens [toff, toff + kTPT)) ----------
    const int cr = tid / kSegs;
    const int seg = tid % kSegs;
    const int toff = seg * kTPT;
    const bool rval = cr < nrows;
    const int64_t rrow = (b * dim + d0 + (rval ? cr : 0)) * (int64_t)L;   // first element of this row
    const float dskip = (rval && p.Dskip) ? p.Dskip[d0 + cr] : 0.f;
    // Row loads issued a chunk ahead: unconditional and left untouched until
    // the next chunk uses them (touching a loaded value waits for it).  A
    // thread's kTPT (1 or 2) tokens are kept raw as one Pair and widened by
    // `rv`, which also gives 0 past the end.  Without z, u's row is read in
    // its place and ignored.
    static_assert(kTPT == 1 || kTPT == 2, "one or two tokens per row thread");
    using Pair = typename std::conditional<sizeof(T) == 2 || kTPT == 1, uint32_t, uint2>::type;
    const T* zl_in = z_in ? z_in : u_in;
    const int64_t blk0 = (b * dim + d0) * (int64_t)L;
    const uint32_t blk_bytes = BUF ? (uint32_t)nrows * (uint32_t)L * (uint32_t)sizeof(T) : 0u;
    const rsrc_t rs_dl = make_rsrc(dl_in + blk0, blk_bytes), rs_u = make_rsrc(u_in + blk0, blk_bytes);
    const rsrc_t rs_go = make_rsrc(go_in + blk0, blk_bytes), rs_z = make_rsrc(zl_in + blk0, blk_bytes);
    auto ld = [&](const T* base, rsrc_t rs, int t) -> Pair {       // tokens t, t + 1 (t even)
        if constexpr (BUF) {
            const uint32_t off = off_if(t < L, ((uint32_t)cr * (uint32_t)L + (uint32_t)t) * (uint32_t)sizeof(T));
            if constexpr (sizeof(T) * kTPT == 2) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
            else if constexpr (sizeof(T) * kTPT == 4) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
            else return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
        } else {
            const T e0 = base[rrow + (t < L ? t : L - 1)];
            if constexpr (kTPT == 1) {
                if constexpr (sizeof(T) == 2) return (uint32_t)e0;
                else return __float_as_uint(e0);
            } else {
                const T e1 = base[rrow + (t + 1 < L ? t + 1 : L - 1)];
                if constexpr (sizeof(T) == 2) return (uint32_t)e0 | ((uint32_t)e1 << 16);
                else return make_uint2(__float_as_uint(e0), __float_as_uint(e1));
            }
        }
    };
    // Store the thread's kTPT values of one output row (BUF: one buffer store;
    // offsets past the sequence or the block's rows are dropped).
    auto st = [&](T* base, int t, const float (&v)[kTPT]) {
        if constexpr (BUF) {
            const rsrc_t rs = make_rsrc(base + blk0, blk_bytes);
            const uint32_t off = off_if(t < L, ((uint32_t)cr * (uint32_t)L + (uint32_t)t) * (uint32_t)sizeof(T));
            if constexpr (sizeof(T) == 2 && kTPT == 1)
                __builtin_amdgcn_raw_buffer_store_b16(to_bf16(v[0]), rs, off, 0, 0);
            else if constexpr (sizeof(T) == 2)
                __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(v[0], v[1]), rs, off, 0, 0);
            else if constexpr (kTPT == 1)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), rs, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(v[0]), __float_as_uint(v[1])}, rs, off, 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < kTPT; ++j)
                if (rval && t + j < L) Elem<T>::store1(base + rrow + t + j, v[j]);
        }
    };
    auto rv = [&](Pair raw, int j, int t) -> float {
        float v;
        if constexpr (sizeof(T) == 2) v = __uint_as_float(j ? (raw & 0xffff0000u) : (raw << 16));
        else if constexpr (kTPT == 1) v = __uint_as_float(raw);
        else v = __uint_as_float(j ? raw.y : raw.x);
        if constexpr (BUF) return v;
        else return (rval && t < L) ? v : 0.f;
    };

    // ================= 1. forward sweep: chunk-start checkpoints =================
    // (delta, u) and B / C of the next line group of chunks are loaded while
    // the last chunk of this group is scanned.
    Pair f_dl[kLG], f_u[kLG];
    T f_bc[kLG][kBPT];
    auto fetch_fwd = [&](int g0) {                // chunks g0 .. g0 + kLG - 1
#pragma unroll
        for (int c = 0; c < kLG; ++c) {
            const int t = (g0 + c) * kTC + toff;
            f_dl[c] = ld(dl_in, rs_dl, t);
            f_u[c] = ld(u_in, rs_u, t);
        }
#pragma unroll
        for (int c = 0; c < kLG; ++c) fetch_bc(g0 + c, f_bc[c]);
    };
    // Staging of chunk ck into buffer ck & 1 (and, at the last chunk of its
    // group, the fetch of the next group); chunk ck + 1 is staged right after
    // chunk ck is scanned, so one barrier per chunk suffices.
    auto stage_fwd = [&](int ck) {
        float dlv[kTPT], uv[kTPT];
        T bcv[kBPT];
        const int c = ck % kLG;
        const Pair pdl = pick(f_dl, c), pu = pick(f_u, c);
#pragma unroll
        for (int j = 0; j < kTPT; ++j) {
            dlv[j] = rv(pdl, j, ck * kTC + toff + j);
            uv[j] = rv(pu, j, ck * kTC + toff + j);
        }
#pragma unroll
        for (int q = 0; q < kBPT; ++q) {
            T col[kLG];
#pragma unroll
            for (int g = 0; g < kLG; ++g) col[g] = f_bc[g][q];
            bcv[q] = pick(col, c);
        }
        if (c == kLG - 1 && ck + 1 < nck) fetch_fwd(ck + 1);
        stage_bc(ck, bcv, ck & 1);
#pragma unroll
        for (int j = 0; j < kTPT; ++j) s_fw[ck & 1][toff + j][cr] = make_float2(dlv[j], dlv[j] * uv[j]);
    };
    // (left out when the forward pass saved the chunk-start states)
    const int nck_fwd = SAVED ? 0 : nck;
    if (nck_fwd > 0) {
        fetch_fwd(0);
        stage_fwd(0);
    }
    for (int ck = 0; ck < nck_fwd; ++ck) {
        if (cval) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                if (w * NS + s < N) *ckpt(ck, s) = h[s];
        }
        __syncthreads();                          // chunk ck staged; buffer (ck + 1) & 1 free
        read_bc(ck & 1);
#pragma unroll
        for (int k = 0; k < kTC; ++k) {
            const float2 q = s_fw[ck & 1][k][cs];
#pragma unroll
            for (int s = 0; s < NS; ++s) h[s] = fmaf(fast_exp2(q.x * a2[s]), h[s], q.y * Bf[s][k]);
        }
        if (ck + 1 < nck_fwd) stage_fwd(ck + 1);
    }
    __syncthreads();                              // the backward sweep reuses the B / C buffers

    // ================= 2. backward sweep, last chunk first =======================
    // The row data and the chunk-start states of the next chunk (ck - 1) are
    // loaded while this one is processed.
    // The row data and B / C of a line group of chunks are loaded while the
    // first chunk of the following group (walked last) is processed; the
    // chunk-start states one chunk ahead.  (Stores need no grouping: L2
    // merges the partial writes of a line, and the bytes written stay the
    // algorithmic ones.)
    float dDacc = 0.f;
    Pair b_dl[kLG], b_u[kLG], b_go[kLG], b_z[kLG];
    T b_bc[kLG][kBPT];
    float b_hc[NS];
    auto fetch_bwd = [&](int g0) {                // chunks g0 .. g0 + kLG - 1
#pragma unroll
        for (int c = 0; c < kLG; ++c) {
            const int t = (g0 + c) * kTC + toff;
            b_dl[c] = ld(dl_in, rs_dl, t);
            b_u[c] = ld(u_in, rs_u, t);
            b_go[c] = ld(go_in, rs_go, t);
            b_z[c] = ld(zl_in, rs_z, t);
        }
#pragma unroll
        for (int c = 0; c < kLG; ++c) fetch_bc(g0 + c, b_bc[c]);
    };
    auto fetch_hc = [&](int ck) {
#pragma unroll
        for (int s = 0; s < NS; ++s) b_hc[s] = *ckpt_in(ck, s);
    };
    if (nck > 0) {
        fetch_bwd((nck - 1) / kLG * kLG);
        fetch_hc(nck - 1);
    }
    // Chunk ck, the c-th of its line group.  With up to 4 states per lane c
    // is a compile-time constant (the loop below runs the chunks of a group
    // as separate copies of this code), so the group's registers are indexed
    // directly; with more states, where registers are short, one copy and
    // selects.
    auto chunk = [&](int ck, auto cc) {
        const int c = index_of(cc);
        const int t0 = ck * kTC;
        const int g0 = ck - c;
        // stage (delta, delta*u, u, g) -- the row thread keeps its own tokens
        float uu[kTPT], zz[kTPT], go[kTPT], gg[kTPT], sgv[kTPT], dlv[kTPT], hc[NS];
        {
            const Pair pdl = sel(b_dl, cc), pu = sel(b_u, cc), pgo = sel(b_go, cc), pz = sel(b_z, cc);
#pragma unroll
            for (int j = 0; j < kTPT; ++j) {
                const int t = t0 + toff + j;
                dlv[j] = rv(pdl, j, t);
                uu[j] = rv(pu, j, t);
                go[j] = rv(pgo, j, t);
                zz[j] = z_in ? rv(pz, j, t) : 0.f;
            }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) hc[s] = (cval && w * NS + s < N) ? b_hc[s] : 0.f;
        T bcv[kBPT];
#pragma unroll
        for (int q = 0; q < kBPT; ++q) {
            T col[kLG];
#pragma unroll
            for (int g = 0; g < kLG; ++g) col[g] = b_bc[g][q];
            bcv[q] = sel(col, cc);
        }
        if (ck > 0) fetch_hc(ck - 1);
        if (c == 0 && ck > 0) fetch_bwd(g0 - kLG);
        stage_bc(ck, bcv, 0);
#pragma unroll
        for (int j = 0; j < kTPT; ++j) {
            // sigmoid(z), kept for dz: g = dout silu(z) = dout z sigmoid(z)
            sgv[j] = __builtin_amdgcn_rcpf(1.f + fast_exp2(-zz[j] * kLog2e));
            gg[j] = z_in ? go[j] * (zz[j] * sgv[j]) : go[j];
            s_tk[toff + j][cr] = make_float4(dlv[j], dlv[j] * uu[j], uu[j], gg[j]);
        }
        __syncthreads();
        read_bc(0);

        // recompute the chunk's states and decay factors (the factors are kept
        // for the walk when registers allow: NS <= 4); per-wave partial
        // outputs to LDS
        constexpr bool kKeepA = NS <= 4;
        float hs[kTC][NS], as[kKeepA ? kTC : 1][NS];
        {
            float hh[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) hh[s] = hc[s];
#pragma unroll
            for (int k = 0; k < kTC; ++k) {
                const float4 q = s_tk[k][cs];
                float yp = 0.f;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const float e = fast_exp2(q.x * a2[s]);
                    if constexpr (kKeepA) as[k][s] = e;
                    hh[s] = fmaf(e, hh[s], q.y * Bf[s][k]);
                    hs[k][s] = hh[s];
                    yp = fmaf(Cf[s][k], hh[s], yp);
                }
                s_y[w][k][cs] = yp;
            }
        }
        __syncthreads();

        // row threads: y, dz, dD
        float dzv[kTPT];
#pragma unroll
        for (int j = 0; j < kTPT; ++j) {
            float y = dskip * uu[j];
#pragma unroll
            for (int q = 0; q < kNW; ++q) y += s_y[q][toff + j][cr];
            const float sg = sgv[j];
            dzv[j] = go[j] * y * (sg * (1.f + zz[j] * (1.f - sg)));
            dDacc = fmaf(gg[j], uu[j], dDacc);
        }
        if (z_in) st(static_cast<T*>(p.dz), t0 + toff, dzv);

        // walk the chunk backwards.  dB / dC of (state s, token k) summed over
        // the wave's 64 channels: value index ((s 2 + c) kTC + k), c 0 for B
        // and 1 for C; s runs to NSP = max(NS, 2), the padding states are 0.
        // The (s, c) values of a token are reduced at once (tree steps 0 ..
        // log2(2 NSP) - 1), leaving rk[k]; the tokens after the walk.
        // Per token, du and ddelta share sum_n lambda_n B_n (du takes it times
        // delta, ddelta times u, once per token), and ddelta and dA share
        // lambda_n a_n h_{t-1,n} (times A_n and delta), which is the carried
        // adjoint a_n lambda_n times h_{t-1,n}.
        float rk[kTC];
#pragma unroll
        for (int k = kTC - 1; k >= 0; --k) {
            const float4 q = s_tk[k][cs];
            float sb = 0.f, ddp = 0.f;
            float v[2 * kNSP];
#pragma unroll
            for (int s = NS; s < kNSP; ++s) v[2 * s] = v[2 * s + 1] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const float bv = Bf[s][k], cv = Cf[s][k];
                const float lt = fmaf(q.w, cv, lam[s]);
                const float hp = k > 0 ? hs[k > 0 ? k - 1 : 0][s] : hc[s];
                float a;
                if constexpr (kKeepA) a = as[k][s];
                else a = fast_exp2(q.x * a2[s]);
                lam[s] = a * lt;                      // a_t lambda_t, carried to token t - 1
                const float pah = lam[s] * hp;        // lambda_t a_t h_{t-1}
                v[2 * s] = lt * q.y;
                v[2 * s + 1] = q.w * hs[k][s];
                sb = fmaf(lt, bv, sb);
                ddp = fmaf(pah, Af[s], ddp);
                dAacc[s] = fmaf(pah, q.x, dAacc[s]);
            }
            tree<0, 2 * kNSP>(v);
            rk[k] = v[0];
            s_p[w][k][cs] = make_float2(q.x * sb, fmaf(q.z, sb, ddp));
        }
        tree<log2i(2 * kNSP), kTC>(rk);
        {
            // this workgroup's partial sums for the chunk: lane L holds the
            // values L R .. L R + R - 1 of the wave's kVPW
            constexpr int R = kVPW / 64;
            float* part = p.part + ((b * nblk_d + dblk) * nck + ck) * (int64_t)(kNW * kVPW) + w * kVPW +
                          cs * R;
            if constexpr (R == 1) part[0] = rk[0];
            else *reinterpret_cast<float2*>(part) = make_float2(rk[0], rk[1]);
        }
        __syncthreads();

        // row threads: du, ddelta
        float duv[kTPT], ddv[kTPT];
#pragma unroll
        for (int j = 0; j < kTPT; ++j) {
            duv[j] = gg[j] * dskip;
            ddv[j] = 0.f;
#pragma unroll
            for (int q = 0; q < kNW; ++q) {
                const float2 v = s_p[q][toff + j][cr];
                duv[j] += v.x;
                ddv[j] += v.y;
            }
        }
        st(static_cast<T*>(p.du), t0 + toff, duv);
        st(static_cast<T*>(p.ddelta), t0 + toff, ddv);
    };
    // groups last first, and in a group its chunks last first (the first
    // group visited may be partial: its chunks past the end are skipped, a
    // test uniform over the workgroup)
    if constexpr (NS <= 4) {
        for (int g0 = nck > 0 ? (nck - 1) / kLG * kLG : -1; g0 >= 0; g0 -= kLG)
            down_for<kLG - 1>([&](auto cc) {
                const int ck = g0 + decltype(cc)::value;
                if (ck < nck) chunk(ck, cc);
            });
    } else {
        for (int ck = nck - 1; ck >= 0; --ck) chunk(ck, ck % kLG);
    }

    // ---- ends: dh0, dA, dD -------------------------------------------------------
    if (cval) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int n = w * NS + s;
            if (n < N) {
                if (p.dh0) p.dh0[ch * N + n] = lam[s];
                atomicAdd(p.dA + (d0 + cs) * N + n, dAacc[s]);
            }
        }
    }
    // dD: the 8 row threads of a channel hold partials over their tokens
#pragma unroll
    for (int m = 1; m < kSegs; m <<= 1) dDacc += __shfl_xor(dDacc, m, 64);
    if (rval && seg == 0 && p.dD) atomicAdd(p.dD + d0 + cr, dDacc);
}

// dB, dC[b, n, t] = sum over the channel blocks of the partial sums.  Per
// (batch, block, chunk) the partials are [wave][(s 2 + c) kTC + k] with
// n = wave NS + s, c 0 for B and 1 for C.
template <int NS>
__global__ void s6_bwd_reduce_bc_kernel(S6BwdParams p) {
    constexpr int kTC = ChunkLen<NS>::value;
    constexpr int kNSP = NS < 2 ? 2 : NS;
    constexpr int kVPW = 2 * kNSP * kTC;
    constexpr int PER = kNW * kVPW;
    const int64_t nblk = (p.dim + 63) / 64;
    const int nck = (p.L + kTC - 1) / kTC;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (b, chunk, j)
    if (i >= p.batch * nck * (int64_t)PER) return;
    const int j = (int)(i % PER);
    const int64_t bc = i / PER;
    const int ck = (int)(bc % nck);
    const int64_t b = bc / nck;
    const int w = j / kVPW, idx = j % kVPW;
    const int k = idx % kTC, sc = idx / kTC;
    const int s = sc >> 1, c = sc & 1;
    const int n = w * NS + s;
    const int t = ck * kTC + k;
    if (s >= NS || n >= p.N || t >= p.L) return;
    // eight loads in flight per step, summed in a fixed order (deterministic)
    const float* src = p.part + (b * nblk * nck + ck) * (int64_t)PER + j;
    const int64_t stride = nck * (int64_t)PER;
    float part[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int64_t blk = 0;
    for (; blk + 8 <= nblk; blk += 8) {
#pragma unroll
        for (int q = 0; q < 8; ++q) part[q] += src[(blk + q) * stride];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
        if (blk + q < nblk) part[q] += src[(blk + q) * stride];
    const float acc = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
    (c ? p.dC : p.dB)[(b * p.N + n) * (int64_t)p.L + t] = acc;
}

__global__ void zero_kernel(float* a, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) a[i] = 0.f;
}

hipError_t zero(float* a, int64_t n, hipStream_t stream) {
    if (!a || n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n);
    return hipGetLastError();
}

template <typename T, int NS>
hipError_t launch_ns(const S6BwdParams& p, hipStream_t stream) {
    const int64_t blocks = ((p.dim + 63) / 64) * p.batch;
    const bool buf = p.L % 2 == 0 && int64_t(64) * p.L * int64_t(sizeof(T)) < (int64_t(1) << 31);
    auto kern = p.saved ? (buf ? s6_scan_bwd_kernel<T, NS, true, true> : s6_scan_bwd_kernel<T, NS, false, true>)
                        : (buf ? s6_scan_bwd_kernel<T, NS, true, false> : s6_scan_bwd_kernel<T, NS, false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kNW * 64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kTC = ChunkLen<NS>::value;
    const int64_t n = p.batch * ((p.L + kTC - 1) / kTC) * (int64_t)(kNW * (NS < 2 ? 2 : NS) * kTC * 2);
    const int64_t rblocks = (n + 255) / 256;
    if (rblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((s6_bwd_reduce_bc_kernel<NS>), dim3((unsigned)rblocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const S6BwdParams& p, hipStream_t stream) {
    if (p.N <= 8) return launch_ns<T, 1>(p, stream);
    if (p.N <= 16) return launch_ns<T, 2>(p, stream);
    if (p.N <= 32) return launch_ns<T, 4>(p, stream);
    return launch_ns<T, 8>(p, stream);
}

}  // namespace

// Workspace: the chunk-start states [batch, chunk, N, dim], then the dB / dC
// partial sums [batch, channel block, chunk, 8 NS states, TC tokens, 2].
static int ns_of(int64_t N) { return N <= 8 ? 1 : N <= 16 ? 2 : N <= 32 ? 4 : 8; }

int64_t s6_bwd_ckpt_floats(int64_t batch, int64_t dim, int64_t L, int64_t N) {
    const int tc = ns_of(N) <= 2 ? ChunkLen<2>::value : ChunkLen<4>::value;
    const int64_t nck = (L + tc - 1) / tc;
    return (batch * nck * N * dim + 63) / 64 * 64;
}

size_t s6_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t L, int64_t N) {
    const int ns = ns_of(N);
    const int tc = ns <= 2 ? ChunkLen<2>::value : ChunkLen<4>::value;
    const int64_t nck = (L + tc - 1) / tc;
    const int64_t part = batch * ((dim + 63) / 64) * nck * (int64_t)(kNW * (ns < 2 ? 2 : ns) * tc * 2);
    return (size_t)(s6_bwd_ckpt_floats(batch, dim, L, N) + part) * sizeof(float);
}

hipError_t launch_s6_scan_bwd(const S6BwdParams& p, bool is_bf16, hipStream_t stream) {
    hipError_t e;
    if ((e = zero(p.dA, p.dim * p.N, stream)) != hipSuccess) return e;
    if ((e = zero(p.dD, p.dD ? p.dim : 0, stream)) != hipSuccess) return e;
    return is_bf16 ? launch_t<uint16_t>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace mssm
