// ssd_general.hip -- Mamba-2 SSD, chunked, for any headdim and d_state up to
// 256, float32 or bfloat16 storage (the sizes the bf16 MFMA kernels of
// ssd.hip do not take).
//
// What it computes ("State-Space Model Optimization Patterns" page, section 2
// "State Space Duality" and section 9 "Chunked Computation"): per batch row
// b, head h (group g = h / (H/G)) and head channel p, with a scalar
// transition per head,
//     H[p,n] <- exp(dt_t*A_h) * H[p,n] + dt_t * x_t[p] * B_t[n]
//     y_t[p]  = (sum_n C_t[n] * H[p,n] + D_h * x_t[p]) * silu(z_t[p]),
// chunk by chunk: within a chunk of K tokens the outputs are the masked
// quadratic form plus the carried-in state,
//     y_i = sum_{j<=i} (C_i . B_j) exp(s_i - s_j) dt_j x_j + exp(s_i) C_i . H_in + D x_i,
// s the running sum of dt*A over the chunk, and the state passed to the next
// chunk is exp(s_end) H_in + sum_j exp(s_end - s_j) dt_j x_j B_j^T.
//
// Design: a workgroup per (b, head, 32 head channels) walks the sequence in
// chunks of K = 32 tokens.  Per chunk it stages dt, x, B and C in LDS as fp32
// (rows of B, C padded with zeros to whole 16-state tiles), forms the running
// sum, then computes the three products on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: fp32 operands and accumulation, so float32 inputs
// keep float32 accuracy), 16 x 16 tiles:
//   scores   M = C B^T     the three tiles on or below the diagonal, masked
//                          and scaled by the decay and dt;
//   outputs  Y = diag(e^s) C H^T + M X    one tile per output wave;
//   state    H = e^{s_end} H + Xw^T B     the state's tiles held in wave
//                          accumulators across chunks (copied to LDS for the
//                          next chunk's C H^T).
// Up to d_state 128 a scores kernel forms C B^T once per (b, chunk, group)
// and an 8-wave two-role kernel does the rest with one barrier pair per
// chunk; above, a 4-wave kernel does all of it in four phases per chunk.  The
// next chunk's inputs are loaded into registers while the current one is
// computed.  The chunk length of the call is a tile size that does not
// change the result beyond rounding; this path always uses 32.
// Every exponent s_i - s_j (j <= i), s_i and s_end - s_j is <= 0 for A_h <= 0,
// so no factor exceeds 1.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mssm {

namespace {

constexpr int kGK = 32;          // chunk length (tokens)
constexpr int kGP = 32;          // head channels per workgroup
constexpr int kGNMax = 256;      // largest d_state
// LDS row strides (floats), 4 mod 32: the 64 lanes of an operand read (16
// rows x 4 columns) then hit every bank exactly twice, the least possible.
constexpr int kRS = kGNMax + 4;  // B, C and the state
constexpr int kXS = kGP + 4;     // x, the scaled x and the scores

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// D = A B + C for one 16 x 16 tile, K = 4: lane l holds A[l % 16][l / 16],
// B[l / 16][l % 16], and D[4 (l / 16) + r][l % 16] in register r.
__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ float ldx(const T* p) { return Elem<T>::load1(p); }

// Four consecutive elements as floats from an address aligned to them.
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const uint16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
}

// Inclusive prefix sum of v over the 32 lanes of each half-wave (shuffles).
__device__ __forceinline__ float scan32(float v, int lane) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        const float u = __shfl_up(v, o, 32);
        if ((lane & 31) >= o) v += u;
    }
    return v;
}

// VEC: B / C rows are whole aligned float4s (N a multiple of 4, aligned
// arrays); otherwise element loads.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void ssd_general_kernel(
    const T* __restrict__ X, const T* __restrict__ DT, const float* __restrict__ Ah, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ Dh, const T* __restrict__ Z, const float* __restrict__ h0,
    T* __restrict__ Y, float* __restrict__ hT, int L, int H, int P, int N, int G) {
    __shared__ __align__(16) float sB[kGK][kRS];
    __shared__ __align__(16) float sC[kGK][kRS];
    __shared__ __align__(16) float sH[kGP][kRS];      // state H[p][n] of this workgroup's head channels
    __shared__ __align__(16) float sX[kGK][kXS];      // x[j][p]
    __shared__ __align__(16) float sXw[kGK][kXS];     // dt_j exp(s_end - s_j) x[j][p]
    __shared__ __align__(16) float sM[kGK][kXS];      // masked scores
    __shared__ float sS[kGK], sDt[kGK], sE[kGK];     // running sum (log2 units), dt, 2^s

    // Blocks are dispatched round-robin over the 8 XCDs; number them so that
    // consecutive ids (the heads of one batch row, which read the same B and
    // C rows) share an XCD and its L2.
    uint32_t lid = blockIdx.x;
    if ((gridDim.x & 7u) == 0u) lid = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int npt = (P + kGP - 1) / kGP;
    const int pt = lid % npt;
    const int bh = lid / npt;
    const int h = bh % H;
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int p0 = pt * kGP;
    const int np = min(kGP, P - p0);
    const int NQ = (N + 15) & ~15;                    // states in whole 16-wide tiles
    const int NT = NQ / 16;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15, lk = l >> 4;               // operand row / column within a tile, k within a step
    const float a2 = Ah[h] * kLog2e;
    const float dskip = Dh ? Dh[h] : 0.f;

    const int64_t xrow = (int64_t)H * P;          // elements per token of x, y, z
    const int64_t brow = (int64_t)G * N;          // elements per token of B, C
    const T* xb = X + b * L * xrow + (int64_t)h * P + p0;
    const T* zb = Z ? Z + b * L * xrow + (int64_t)h * P + p0 : nullptr;
    T* yb = Y + b * L * xrow + (int64_t)h * P + p0;
    const T* Bb = Bm + b * L * brow + (int64_t)g * N;
    const T* Cb = Cm + b * L * brow + (int64_t)g * N;
    const T* dtb = DT + b * (int64_t)L * H + h;

    // The state's tiles: tile t = (channel block t & 1, state block t >> 1),
    // wave w holds tiles w, w + 4, ...  (at most 8), lane l register r at
    // channel 16 (t & 1) + 4 lk + r, state 16 (t >> 1) + lr.
    constexpr int kMaxT = 2 * (kGNMax / 16) / 4;
    f32x4_t acc_h[kMaxT];
#pragma unroll
    for (int m = 0; m < kMaxT; ++m) {
        const int t = w + 4 * m;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * (t & 1) + 4 * lk + r, n = 16 * (t >> 1) + lr;
            acc_h[m][r] = (h0 && t < 2 * NT && c < np && n < N) ? h0[((b * H + h) * (int64_t)P + p0 + c) * N + n]
                                                                : 0.f;
        }
    }
    auto write_state = [&]() {
#pragma unroll
        for (int m = 0; m < kMaxT; ++m) {
            const int t = w + 4 * m;
            if (t < 2 * NT) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sH[16 * (t & 1) + 4 * lk + r][16 * (t >> 1) + lr] = acc_h[m][r];
            }
        }
    };
    write_state();
    // the scores tile above the diagonal is never written: zero once
    for (int e = tid; e < 16 * 16; e += 256) sM[e >> 4][16 + (e & 15)] = 0.f;

    // The next chunk's dt, x, z, B and C are loaded into registers while this
    // one is computed.  Every load is issued unconditionally from a clamped
    // address (a branch around a load would make the compiler wait for all
    // loads in flight at the join) and kept raw; the values out of range are
    // replaced by 0 when they are staged, a chunk later (a select right after
    // the load could be rewritten as a load from a selected address, which
    // would put the zero in scratch memory).
    const int xj = tid >> 3, xp = 4 * (tid & 7);  // x: token xj, channels xp .. xp + 3
    const int bq = tid & 63;                      // B / C: float4 bq of rows (tid >> 6) + 4 m
    // this wave's output tile: tokens 16 ob + 4 lk + r, channel 16 oc + lr
    const int ob = w >> 1, oc = w & 1;
    float r_dt = 0.f, r_x[4], r_z[4];
    float4 r_b[8], r_c[8];
    auto fetch = [&](int t0) {
        r_dt = ldx(dtb + (int64_t)min(t0 + tid, L - 1) * H);
        {
            const T* src = xb + (int64_t)min(t0 + xj, L - 1) * xrow;
#pragma unroll
            for (int k = 0; k < 4; ++k) r_x[k] = ldx(src + min(xp + k, np - 1));
        }
        if (zb) {                                 // the gate of this lane's outputs (a uniform branch)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                r_z[r] = ldx(zb + (int64_t)min(t0 + 16 * ob + 4 * lk + r, L - 1) * xrow + min(16 * oc + lr, np - 1));
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int64_t ro = (int64_t)min(t0 + (tid >> 6) + 4 * m, L - 1) * brow;
            if constexpr (VEC) {
                const int64_t o = ro + min(4 * bq, N - 4);
                r_b[m] = ld4(Bb + o);
                r_c[m] = ld4(Cb + o);
            } else {
                float eb[4], ec[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int64_t o = ro + min(4 * bq + k, N - 1);
                    eb[k] = ldx(Bb + o);
                    ec[k] = ldx(Cb + o);
                }
                r_b[m] = make_float4(eb[0], eb[1], eb[2], eb[3]);
                r_c[m] = make_float4(ec[0], ec[1], ec[2], ec[3]);
            }
        }
    };

    if (L > 0) fetch(0);
    for (int t0 = 0; t0 < L; t0 += kGK) {
        const int nt = min(kGK, L - t0);
        __syncthreads();                          // previous chunk done with every buffer
        // ---- stage: dt and the running sum (first half-wave), x, B, C ----
        if (tid < 32) {
            const float dt = tid < nt ? r_dt : 0.f;
            const float s = scan32(dt * a2, tid);
            sDt[tid] = dt;
            sS[tid] = s;
            sE[tid] = fast_exp2(s);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) sX[xj][xp + k] = (xj < nt && xp + k < np) ? r_x[k] : 0.f;
        if (4 * bq < NQ) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int j = (tid >> 6) + 4 * m;
                float4 vb = r_b[m], vc = r_c[m];
                if (j >= nt) vb = vc = make_float4(0.f, 0.f, 0.f, 0.f);
                if (4 * bq + 1 > N) vb.x = vc.x = 0.f;   // columns past N (padding of the last tile)
                if (4 * bq + 2 > N) vb.y = vc.y = 0.f;
                if (4 * bq + 3 > N) vb.z = vc.z = 0.f;
                if (4 * bq + 4 > N) vb.w = vc.w = 0.f;
                *reinterpret_cast<float4*>(&sB[j][4 * bq]) = vb;
                *reinterpret_cast<float4*>(&sC[j][4 * bq]) = vc;
            }
        }
        float z_cur[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) z_cur[r] = zb ? r_z[r] : 0.f;
        if (t0 + kGK < L) fetch(t0 + kGK);
        __syncthreads();
        const float send = sS[kGK - 1];           // tokens past the end have dt = 0
        if (w < 3) {
            // ---- scores: tile (ti, tj) = (0, 0), (1, 0), (1, 1) ----
            const int ti = w == 0 ? 0 : 1, tj = w == 2 ? 1 : 0;
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;    // two chains over the states
#pragma unroll 4
            for (int k0 = 0; k0 < NQ; k0 += 8) {
                s0 = mfma4(sC[16 * ti + lr][k0 + lk], sB[16 * tj + lr][k0 + lk], s0);
                s1 = mfma4(sC[16 * ti + lr][k0 + 4 + lk], sB[16 * tj + lr][k0 + 4 + lk], s1);
            }
            const int j = 16 * tj + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + 4 * lk + r;
                sM[i][j] = j <= i ? (s0[r] + s1[r]) * fast_exp2(sS[i] - sS[j]) * sDt[j] : 0.f;
            }
        } else {
            // ---- scaled inputs of the state update ----
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = 2 * e + (l >> 5), p = l & 31;
                sXw[j][p] = sDt[j] * fast_exp2(send - sS[j]) * sX[j][p];
            }
        }
        __syncthreads();
        // ---- outputs: this wave's tile ----
        {
            f32x4_t y0 = {0.f, 0.f, 0.f, 0.f}, y1 = y0;
#pragma unroll 4
            for (int k0 = 0; k0 < NQ; k0 += 8) {          // C H^T
                y0 = mfma4(sC[16 * ob + lr][k0 + lk], sH[16 * oc + lr][k0 + lk], y0);
                y1 = mfma4(sC[16 * ob + lr][k0 + 4 + lk], sH[16 * oc + lr][k0 + 4 + lk], y1);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) y0[r] = (y0[r] + y1[r]) * sE[16 * ob + 4 * lk + r];
            // + M X (M is zero past the diagonal tile: 16 or 32 tokens)
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4) y0 = mfma4(sM[16 * ob + lr][k0 + lk], sX[k0 + lk][16 * oc + lr], y0);
            if (ob) {
#pragma unroll
                for (int k0 = 16; k0 < 32; k0 += 4)
                    y0 = mfma4(sM[16 * ob + lr][k0 + lk], sX[k0 + lk][16 * oc + lr], y0);
            }
            const int p = 16 * oc + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ob + 4 * lk + r;
                float out = y0[r] + dskip * sX[i][p];
                if (zb) out *= silu(z_cur[r]);
                if (i < nt && p < np) Elem<T>::store1(yb + (int64_t)(t0 + i) * xrow + p, out);
            }
        }
        __syncthreads();                          // every C H^T has read the old state
        // ---- state: H = 2^send H + Xw^T B, this wave's tiles ----
        {
            const float ed = fast_exp2(send);
#pragma unroll
            for (int m = 0; m < kMaxT; ++m) {
                const int t = w + 4 * m;
                if (t < 2 * NT) {
                    const int cb = t & 1, sb = t >> 1;
                    f32x4_t acc = acc_h[m] * ed;
#pragma unroll
                    for (int k0 = 0; k0 < kGK; k0 += 4)
                        acc = mfma4(sXw[k0 + lk][16 * cb + lr], sB[k0 + lk][16 * sb + lr], acc);
                    acc_h[m] = acc;
                }
            }
            write_state();
        }
    }
    if (hT) {
#pragma unroll
        for (int m = 0; m < kMaxT; ++m) {
            const int t = w + 4 * m;
            if (t < 2 * NT) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int c = 16 * (t & 1) + 4 * lk + r, n = 16 * (t >> 1) + lr;
                    if (c < np && n < N) hT[((b * H + h) * (int64_t)P + p0 + c) * N + n] = acc_h[m][r];
                }
            }
        }
    }
}

// d_state up to 128 (the scores kernel and the two-role kernel below).
constexpr int kRNMax = 128;      // largest d_state of the two-role kernel
constexpr int kRRS = kRNMax + 4; // B, C and state row stride, 4 mod 32 as above

// The raw scores G = C B^T of every 32-token chunk, per (b, chunk, group):
// they depend on the group only, so the two-role kernel below reads them
// instead of recomputing them for every head and channel block.  Waves 0-2
// form the tiles (0, 0), (1, 0), (1, 1) (the one above the diagonal is never
// used) and store each as the accumulator fragments the MFMA leaves: lane l
// of tile t writes its four registers as one float4 at
//   ws[((b * nch + chunk) * G + g) * 1024 + 256 t + 4 l],
// so the reader of tile t loads exactly its own registers, 16 contiguous bytes
// per lane.  Rows past the sequence and states past N are zero.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void ssd_general_scores_kernel(const T* __restrict__ Bm, const T* __restrict__ Cm,
                                                                 float* __restrict__ ws, int L, int N, int G, int nch) {
    __shared__ __align__(16) float sB[kGK][kRRS];
    __shared__ __align__(16) float sC[kGK][kRRS];
    const int g = blockIdx.x % G;
    const int c = (blockIdx.x / G) % nch;
    const int64_t b = blockIdx.x / ((int64_t)G * nch);
    const int t0 = c * kGK, nt = min(kGK, L - t0);
    const int NQ = (N + 15) & ~15;
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lk = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t brow = (int64_t)G * N;
    const T* Bb = Bm + b * L * brow + (int64_t)g * N;
    const T* Cb = Cm + b * L * brow + (int64_t)g * N;
    const int bq = tid & 31;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int j = (tid >> 5) + 8 * m;
        if (4 * bq < NQ) {
            const int64_t ro = (int64_t)min(t0 + j, L - 1) * brow;
            float4 vb, vc;
            if constexpr (VEC) {
                vb = ld4(Bb + ro + min(4 * bq, N - 4));
                vc = ld4(Cb + ro + min(4 * bq, N - 4));
            } else {
                float eb[4], ec[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    eb[k] = ldx(Bb + ro + min(4 * bq + k, N - 1));
                    ec[k] = ldx(Cb + ro + min(4 * bq + k, N - 1));
                }
                vb = make_float4(eb[0], eb[1], eb[2], eb[3]);
                vc = make_float4(ec[0], ec[1], ec[2], ec[3]);
            }
            if (j >= nt) vb = vc = make_float4(0.f, 0.f, 0.f, 0.f);
            if (4 * bq + 1 > N) vb.x = vc.x = 0.f;
            if (4 * bq + 2 > N) vb.y = vc.y = 0.f;
            if (4 * bq + 3 > N) vb.z = vc.z = 0.f;
            if (4 * bq + 4 > N) vb.w = vc.w = 0.f;
            *reinterpret_cast<float4*>(&sB[j][4 * bq]) = vb;
            *reinterpret_cast<float4*>(&sC[j][4 * bq]) = vc;
        }
    }
    __syncthreads();
    if (w < 3) {
        const int ti = w == 0 ? 0 : 1, tj = w == 2 ? 1 : 0;
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
        for (int k0 = 0; k0 < NQ; k0 += 8) {
            s0 = mfma4(sC[16 * ti + lr][k0 + lk], sB[16 * tj + lr][k0 + lk], s0);
            s1 = mfma4(sC[16 * ti + lr][k0 + 4 + lk], sB[16 * tj + lr][k0 + 4 + lk], s1);
        }
        const f32x4_t sc = s0 + s1;
        *reinterpret_cast<float4*>(ws + (int64_t)blockIdx.x * 1024 + 256 * w + 4 * l) =
            make_float4(sc[0], sc[1], sc[2], sc[3]);
    }
}

// d_state up to 128: the same chunk computation with 8 waves in two roles
// and the LDS buffers doubled by chunk parity, so that each chunk needs two
// barriers and two kinds of work overlap in each phase.  Waves 0-3 (one per
// SIMD) mask a chunk's scores (read from the scores kernel's workspace) and
// scale its inputs, then compute its outputs; waves 4-7 hold the state, load
// and stage the inputs.  Chunk c:
//   phase A  waves 0-2: masked scores of chunk c; wave 3: Xw of chunk c
//            waves 4-7: state update of chunk c-1 (H entering chunk c)
//   phase B  waves 0-3: outputs of chunk c (its C, that H, its scores and x)
//            waves 4-7: stage chunk c+1 into the other buffers, then issue
//            the loads of chunk c+2
// Each buffer is written in one phase and read in later phases only, before
// the buffer of the same parity is written again (two chunks later).

// KQ: the columns C H^T runs over, NQ rounded up to 32, 64 or 128 (the
// columns past NQ are zero), so that its loop has a fixed length and its LDS
// reads can be issued ahead of the products.
template <typename T, bool VEC, int KQ>
__global__ __launch_bounds__(512) void ssd_general_roles_kernel(
    const T* __restrict__ X, const T* __restrict__ DT, const float* __restrict__ Ah, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ Dh, const T* __restrict__ Z, const float* __restrict__ h0,
    T* __restrict__ Y, float* __restrict__ hT, const float* __restrict__ Gs, int L, int H, int P, int N, int G) {
    __shared__ __align__(16) float sB[2][kGK][kRRS];
    __shared__ __align__(16) float sC[2][kGK][kRRS];
    __shared__ __align__(16) float sH[kGP][kRRS];      // state entering the chunk, H[p][n]
    __shared__ __align__(16) float sX[2][kGK][kXS];
    __shared__ __align__(16) float sXw[2][kGK][kXS];   // dt_j exp(s_end - s_j) x[j][p]
    __shared__ __align__(16) float sM[2][kGK][kXS];    // masked scores, by chunk parity
    __shared__ float sS[2][kGK], sDt[2][kGK], sE[2][kGK];

    uint32_t lid = blockIdx.x;
    if ((gridDim.x & 7u) == 0u) lid = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int npt = (P + kGP - 1) / kGP;
    const int pt = lid % npt;
    const int bh = lid / npt;
    const int h = bh % H;
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int p0 = pt * kGP;
    const int np = min(kGP, P - p0);
    const int NQ = (N + 15) & ~15;
    const int NT = NQ / 16;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15, lk = l >> 4;
    const float a2 = Ah[h] * kLog2e;
    const float dskip = Dh ? Dh[h] : 0.f;
    const int nch = (L + kGK - 1) / kGK;

    const int64_t xrow = (int64_t)H * P;
    const int64_t brow = (int64_t)G * N;
    const T* xb = X + b * L * xrow + (int64_t)h * P + p0;
    const T* zb = Z ? Z + b * L * xrow + (int64_t)h * P + p0 : nullptr;
    T* yb = Y + b * L * xrow + (int64_t)h * P + p0;
    const T* Bb = Bm + b * L * brow + (int64_t)g * N;
    const T* Cb = Cm + b * L * brow + (int64_t)g * N;
    const T* dtb = DT + b * (int64_t)L * H + h;

    for (int e = tid; e < 2 * 16 * 16; e += 512) sM[e >> 8][(e >> 4) & 15][16 + (e & 15)] = 0.f;   // above the diagonal, never written
    for (int e = tid; e < kGK * KQ; e += 512) {   // columns NQ .. KQ of C and H: zero, never written
        const int r = e / KQ, k = e % KQ;
        if (k >= NQ) sC[0][r][k] = sC[1][r][k] = sH[r][k] = 0.f;
    }

    if (w < 4) {
        // ======== waves 0-3: scores, scaled inputs, outputs ========
        // The outputs of chunk c are formed in two halves: C H^T (which needs
        // the state entering the chunk) in phase B of chunk c, and the rest
        // (M X, skip, gate, store) in phase A of chunk c + 1, beside the next
        // chunk's masking.  Each phase then holds about as much work for
        // these waves as for the state waves.
        const int ob = w >> 1, oc = w & 1;        // output tile: tokens 16 ob + 4 lk + r, channel 16 oc + lr
        float r_z[4] = {0.f, 0.f, 0.f, 0.f};
        float4 r_g = make_float4(0.f, 0.f, 0.f, 0.f);
        const float* gsb = Gs + ((b * nch) * G + g) * 1024 + 256 * min(w, 2) + 4 * l;   // this wave's tile, chunk 0
        auto fetch_o = [&](int t0) {              // this wave's raw scores and gate values of a chunk
            if (w < 3) r_g = *reinterpret_cast<const float4*>(gsb + (int64_t)(t0 / kGK) * G * 1024);
            if (zb) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    r_z[r] = ldx(zb + (int64_t)min(t0 + 16 * ob + 4 * lk + r, L - 1) * xrow + min(16 * oc + lr, np - 1));
            }
        };
        f32x4_t yo = {0.f, 0.f, 0.f, 0.f};        // C H^T of the pending chunk, rows scaled by 2^s
        float z_pend[4] = {0.f, 0.f, 0.f, 0.f};   // its gate values
        // the pending chunk cp's outputs: + M X (M is zero past the diagonal
        // tile: 16 or 32 tokens, two chains), skip, gate, store
        auto finish = [&](int cp) {
            const int t0 = cp * kGK, nt = min(kGK, L - t0), pi = cp & 1;
            f32x4_t y0 = yo, ym = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 8) {
                y0 = mfma4(sM[pi][16 * ob + lr][k0 + lk], sX[pi][k0 + lk][16 * oc + lr], y0);
                ym = mfma4(sM[pi][16 * ob + lr][k0 + 4 + lk], sX[pi][k0 + 4 + lk][16 * oc + lr], ym);
            }
            if (ob) {
#pragma unroll
                for (int k0 = 16; k0 < 32; k0 += 8) {
                    y0 = mfma4(sM[pi][16 * ob + lr][k0 + lk], sX[pi][k0 + lk][16 * oc + lr], y0);
                    ym = mfma4(sM[pi][16 * ob + lr][k0 + 4 + lk], sX[pi][k0 + 4 + lk][16 * oc + lr], ym);
                }
            }
            y0 += ym;
            const int p = 16 * oc + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ob + 4 * lk + r;
                float out = y0[r] + dskip * sX[pi][i][p];
                if (zb) out *= silu(z_pend[r]);
                if (i < nt && p < np) Elem<T>::store1(yb + (int64_t)(t0 + i) * xrow + p, out);
            }
        };
        fetch_o(0);
        __syncthreads();                          // chunk 0 staged, the initial state in sH
        for (int c = 0; c < nch; ++c) {
            const int t0 = c * kGK, pi = c & 1;
            // ---- phase A: the previous chunk's outputs; this chunk's masked scores and Xw ----
            if (c > 0) finish(c - 1);
            if (w < 3) {
                const int ti = w == 0 ? 0 : 1, tj = w == 2 ? 1 : 0;
                const float sc[4] = {r_g.x, r_g.y, r_g.z, r_g.w};
                const int j = 16 * tj + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * ti + 4 * lk + r;
                    sM[pi][i][j] = j <= i ? sc[r] * fast_exp2(sS[pi][i] - sS[pi][j]) * sDt[pi][j] : 0.f;
                }
            } else {
                const float send = sS[pi][kGK - 1];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = 2 * e + (l >> 5), p = l & 31;
                    sXw[pi][j][p] = sDt[pi][j] * fast_exp2(send - sS[pi][j]) * sX[pi][j][p];
                }
            }
            __syncthreads();
            // ---- phase B: C H^T of this chunk (the state entering it is in sH) ----
            {
                // C H^T over KQ columns: lane group lk takes the columns
                // [lk KQ/4, (lk + 1) KQ/4) in order (any assignment of columns
                // to (step, lane group) sums the same products), so a lane reads
                // its operands as 16-byte runs
                constexpr int KL = KQ / 4;
                const float* ca = &sC[pi][16 * ob + lr][lk * KL];
                const float* ha = &sH[16 * oc + lr][lk * KL];
                f32x4_t y0 = {0.f, 0.f, 0.f, 0.f}, y1 = y0;
#pragma unroll
                for (int q = 0; q < KL; q += 4) {
                    const float4 av = *reinterpret_cast<const float4*>(ca + q);
                    const float4 hv = *reinterpret_cast<const float4*>(ha + q);
                    y0 = mfma4(av.x, hv.x, y0);
                    y1 = mfma4(av.y, hv.y, y1);
                    y0 = mfma4(av.z, hv.z, y0);
                    y1 = mfma4(av.w, hv.w, y1);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) yo[r] = (y0[r] + y1[r]) * sE[pi][16 * ob + 4 * lk + r];
#pragma unroll
                for (int r = 0; r < 4; ++r) z_pend[r] = r_z[r];
                if (c + 1 < nch) fetch_o(t0 + kGK);
            }
            __syncthreads();
        }
        if (nch > 0) finish(nch - 1);
        __syncthreads();                          // the last state update (waves 4-7)
    } else {
        // ======== waves 4-7: the state; loads and staging ========
        const int st = tid - 256;                 // 0 .. 255
        const int ws = w - 4;
        // state tiles t = ws + 4 m: channel block t & 1, state block t >> 1;
        // lane register r at channel 16 (t & 1) + 4 lk + r, state 16 (t >> 1) + lr
        constexpr int kMT = 2 * (kRNMax / 16) / 4;
        f32x4_t acc_h[kMT];
#pragma unroll
        for (int m = 0; m < kMT; ++m) {
            const int t = ws + 4 * m;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * (t & 1) + 4 * lk + r, n = 16 * (t >> 1) + lr;
                acc_h[m][r] = (h0 && t < 2 * NT && c < np && n < N)
                                  ? h0[((b * H + h) * (int64_t)P + p0 + c) * N + n] : 0.f;
            }
        }
        auto write_state = [&]() {
#pragma unroll
            for (int m = 0; m < kMT; ++m) {
                const int t = ws + 4 * m;
                if (t < 2 * NT) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sH[16 * (t & 1) + 4 * lk + r][16 * (t >> 1) + lr] = acc_h[m][r];
                }
            }
        };
        // H <- 2^send H + Xw^T B for chunk c (buffers of parity c & 1).  The
        // wave's valid tiles (all in channel block ws & 1, so they share the
        // A operand) are independent accumulation chains, interleaved.
        const int nvt = (2 * NT - ws + 3) >> 2;       // valid tiles of this wave (uniform)
        auto update_tiles = [&](auto mc, int pi, float ed) {
            constexpr int M = decltype(mc)::value;
            f32x4_t acc[M];
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m] = acc_h[m] * ed;
#pragma unroll
            for (int k0 = 0; k0 < kGK; k0 += 4) {
                const float a = sXw[pi][k0 + lk][16 * (ws & 1) + lr];
                float bv[M];
#pragma unroll
                for (int m = 0; m < M; ++m) bv[m] = sB[pi][k0 + lk][16 * ((ws >> 1) + 2 * m) + lr];
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m] = mfma4(a, bv[m], acc[m]);
            }
#pragma unroll
            for (int m = 0; m < M; ++m) acc_h[m] = acc[m];
        };
        auto state_update = [&](int c) {
            const int pi = c & 1;
            const float ed = fast_exp2(sS[pi][kGK - 1]);
            switch (nvt) {
                case 4: update_tiles(std::integral_constant<int, 4>{}, pi, ed); break;
                case 3: update_tiles(std::integral_constant<int, 3>{}, pi, ed); break;
                case 2: update_tiles(std::integral_constant<int, 2>{}, pi, ed); break;
                case 1: update_tiles(std::integral_constant<int, 1>{}, pi, ed); break;
                default: break;
            }
        };
        // loads of a chunk (clamped addresses, unconditional; zeroed at staging)
        const int xj = st >> 3, xp = 4 * (st & 7);   // x: token xj, channels xp .. xp + 3
        const int bq = st & 31;                       // B / C: float4 bq of rows (st >> 5) + 8 m
        float r_dt = 0.f, r_x[4];
        float4 r_b[4], r_c[4];
        auto fetch = [&](int t0) {
            r_dt = ldx(dtb + (int64_t)min(t0 + (st & 31), L - 1) * H);
            {
                const T* src = xb + (int64_t)min(t0 + xj, L - 1) * xrow;
#pragma unroll
                for (int k = 0; k < 4; ++k) r_x[k] = ldx(src + min(xp + k, np - 1));
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int64_t ro = (int64_t)min(t0 + (st >> 5) + 8 * m, L - 1) * brow;
                if constexpr (VEC) {
                    const int64_t o = ro + min(4 * bq, N - 4);
                    r_b[m] = ld4(Bb + o);
                    r_c[m] = ld4(Cb + o);
                } else {
                    float eb[4], ec[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int64_t o = ro + min(4 * bq + k, N - 1);
                        eb[k] = ldx(Bb + o);
                        ec[k] = ldx(Cb + o);
                    }
                    r_b[m] = make_float4(eb[0], eb[1], eb[2], eb[3]);
                    r_c[m] = make_float4(ec[0], ec[1], ec[2], ec[3]);
                }
            }
        };
        auto stage = [&](int c) {
            const int t0 = c * kGK, nt = min(kGK, L - t0), pi = c & 1;
            if (st < 32) {                        // wave 4, lanes 0-31: dt and the running sum
                const float dt = st < nt ? r_dt : 0.f;
                const float s = scan32(dt * a2, st);
                sDt[pi][st] = dt;
                sS[pi][st] = s;
                sE[pi][st] = fast_exp2(s);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) sX[pi][xj][xp + k] = (xj < nt && xp + k < np) ? r_x[k] : 0.f;
            if (4 * bq < NQ) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int j = (st >> 5) + 8 * m;
                    float4 vb = r_b[m], vc = r_c[m];
                    if (j >= nt) vb = vc = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (4 * bq + 1 > N) vb.x = vc.x = 0.f;
                    if (4 * bq + 2 > N) vb.y = vc.y = 0.f;
                    if (4 * bq + 3 > N) vb.z = vc.z = 0.f;
                    if (4 * bq + 4 > N) vb.w = vc.w = 0.f;
                    *reinterpret_cast<float4*>(&sB[pi][j][4 * bq]) = vb;
                    *reinterpret_cast<float4*>(&sC[pi][j][4 * bq]) = vc;
                }
            }
        };
        write_state();
        fetch(0);
        stage(0);
        if (nch > 1) fetch(kGK);
        __syncthreads();                          // chunk 0 staged, the initial state in sH
        for (int c = 0; c < nch; ++c) {
            // ---- phase A: the state entering chunk c ----
            if (c > 0) {
                state_update(c - 1);
                write_state();
            }
            __syncthreads();
            // ---- phase B: stage chunk c + 1, load chunk c + 2 ----
            if (c + 1 < nch) {
                stage(c + 1);
                if (c + 2 < nch) fetch((c + 2) * kGK);
            }
            __syncthreads();
        }
        if (nch > 0) state_update(nch - 1);
        __syncthreads();
        if (hT) {
#pragma unroll
            for (int m = 0; m < kMT; ++m) {
                const int t = ws + 4 * m;
                if (t < 2 * NT) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int c = 16 * (t & 1) + 4 * lk + r, n = 16 * (t >> 1) + lr;
                        if (c < np && n < N) hT[((b * H + h) * (int64_t)P + p0 + c) * N + n] = acc_h[m][r];
                    }
                }
            }
        }
    }
}

}  // namespace

bool ssd_general_supported(int64_t P, int64_t N) { return P >= 1 && N >= 1 && N <= kGNMax; }

size_t ssd_general_workspace_bytes(int64_t batch, int64_t L, int64_t N, int64_t G) {
    if (N > kRNMax) return 0;                     // the wide kernel forms its scores itself
    return (size_t)(batch * ((L + kGK - 1) / kGK) * G * 1024 * (int64_t)sizeof(float));
}

hipError_t launch_ssd_general(const SSDParams& p, bool is_bf16, hipStream_t stream) {
    const int64_t blocks = p.batch * p.H * ((p.P + kGP - 1) / kGP);
    const int nch = (p.L + kGK - 1) / kGK;
    const int64_t sblocks = p.batch * nch * p.G;
    if (blocks > INT32_MAX || sblocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const uintptr_t align = (is_bf16 ? 8 : 16) - 1;
    const bool vec = p.N % 4 == 0 && ((reinterpret_cast<uintptr_t>(p.Bm) | reinterpret_cast<uintptr_t>(p.Cm)) & align) == 0;
    const bool roles = p.N <= kRNMax;
    float* gs = static_cast<float*>(p.workspace);
    auto run = [&](auto tag) -> hipError_t {
        using E = decltype(tag);
        const E* Bm = static_cast<const E*>(p.Bm);
        const E* Cm = static_cast<const E*>(p.Cm);
        if (roles) {
            auto sk = vec ? ssd_general_scores_kernel<E, true> : ssd_general_scores_kernel<E, false>;
            hipLaunchKernelGGL(sk, dim3((unsigned)sblocks), dim3(256), 0, stream, Bm, Cm, gs, p.L, p.N, p.G, nch);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int nq = (p.N + 15) & ~15;
            auto pick = [&](auto kq) {
                constexpr int KQ = decltype(kq)::value;
                return vec ? ssd_general_roles_kernel<E, true, KQ> : ssd_general_roles_kernel<E, false, KQ>;
            };
            auto kern = nq <= 32 ? pick(std::integral_constant<int, 32>{})
                                 : nq <= 64 ? pick(std::integral_constant<int, 64>{})
                                            : pick(std::integral_constant<int, 128>{});
            hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(512), 0, stream, static_cast<const E*>(p.x),
                               static_cast<const E*>(p.dt), p.A, Bm, Cm, p.Dskip, static_cast<const E*>(p.z), p.h0,
                               static_cast<E*>(p.y), p.h_final, static_cast<const float*>(gs), p.L, p.H, p.P, p.N,
                               p.G);
        } else {
            auto kern = vec ? ssd_general_kernel<E, true> : ssd_general_kernel<E, false>;
            hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const E*>(p.x),
                               static_cast<const E*>(p.dt), p.A, Bm, Cm, p.Dskip, static_cast<const E*>(p.z), p.h0,
                               static_cast<E*>(p.y), p.h_final, p.L, p.H, p.P, p.N, p.G);
        }
        return hipGetLastError();
    };
    return is_bf16 ? run(uint16_t{}) : run(float{});
}

}  // namespace mssm
