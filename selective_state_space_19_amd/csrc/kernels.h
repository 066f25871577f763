// kernels.h -- internal launchers of libmssm (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

struct S6Params {
    const void* u;
    const void* delta;
    const void* Bm;
    const void* Cm;
    const void* z;        // nullable
    const float* A;
    const float* Dskip;   // nullable
    const float* h0;      // nullable
    void* y;
    float* h_final;       // nullable
    int64_t batch, dim;
    int32_t L, N;
    float* ckpt;          // nullable: the states at every backward-chunk start, in the backward's workspace layout
};

// Front end of the scan: u = silu(causal depthwise conv1d(x)) with K taps
// (K <= 4) and delta = softplus(delta_raw + delta_bias).
struct S6FrontEnd {
    const float* conv_w;      // [dim, K]
    const float* conv_b;      // nullable, [dim]
    const void* conv_init;    // nullable, [batch, dim, K - 1] (input dtype)
    const float* delta_bias;  // nullable, [dim]
    int32_t K;
};

struct S6BwdParams {
    const void *u, *delta, *Bm, *Cm, *z, *dout;   // [batch, dim, L] / [batch, N, L] (input dtype)
    const float *A, *Dskip, *h0, *dhT;            // A [dim, N]; Dskip [dim]; h0, dhT [batch, dim, N]
    void *du, *ddelta, *dz;                       // [batch, dim, L] (input dtype)
    float *dA, *dB, *dC, *dD, *dh0;               // fp32: [dim, N], [batch, N, L] x 2, [dim], [batch, dim, N]
    float* ws;                                    // chunk-start states
    float* part;                                  // dB / dC partial sums per channel block
    int64_t batch, dim;
    int32_t L, N;
    int32_t saved;                                // ws already holds the chunk-start states (from the forward)
};

struct SUParams {
    float* state;
    const void* u;
    const void* delta;
    const void* Bm;
    const void* Cm;
    const void* z;        // nullable
    const float* A;
    const float* Dskip;   // nullable
    void* y;
    int64_t batch, dim;
    int32_t N;
};

struct SSDParams {
    const void* x;
    const void* dt;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;   // nullable
    const void* z;        // nullable
    const float* h0;      // nullable
    void* y;
    float* h_final;       // nullable
    void* workspace;
    int64_t batch;
    int32_t L, H, P, N, G, Q;
};

struct SSDUParams {
    float* state;         // [batch, H, P, N] fp32, in place
    const void* x;        // [batch, H, P]
    const void* dt;       // [batch, H]
    const float* A;       // [H]
    const void* Bm;       // [batch, G, N]
    const void* Cm;       // [batch, G, N]
    const float* Dskip;   // nullable, [H]
    const void* z;        // nullable, [batch, H, P]
    void* y;              // [batch, H, P]
    int64_t batch;
    int32_t H, P, N, G;
};

// Each returns hipSuccess or the launch error; is_bf16 selects the storage type.
hipError_t launch_s6_scan(const S6Params& p, bool is_bf16, bool zoh, hipStream_t stream);   // zoh: hold input term
// Only the backward pass's chunk-start states (p.ckpt), as the forward with
// saving would store them; nothing else is read beyond u, delta, A, B, h0 or
// written.
hipError_t launch_s6_save_states(const S6Params& p, bool is_bf16, hipStream_t stream);
hipError_t launch_s6_scan_fused(const S6Params& p, const S6FrontEnd& fe, bool is_bf16, hipStream_t stream);
hipError_t launch_state_update(const SUParams& p, bool is_bf16, hipStream_t stream);
// Backward of the scan; zeroes dA and dD and then accumulates into them.
hipError_t launch_s6_scan_bwd(const S6BwdParams& p, bool is_bf16, hipStream_t stream);
size_t s6_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t L, int64_t N);
int64_t s6_bwd_ckpt_floats(int64_t batch, int64_t dim, int64_t L, int64_t N);  // offset of the partials
// Mamba-2 SSD on the bf16 matrix cores (bf16 storage): the sizes it
// implements (headdim a multiple of 32, d_state 32 / 64 / 128 / 256, chunk
// 64 / 128 / 256, 32-bit offsets within a batch row) and its workspace.
hipError_t launch_ssd_fast(const SSDParams& p, hipStream_t stream);
size_t ssd_fast_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q);
bool ssd_fast_supported(int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q);
// Mamba-2 SSD on the fp32 matrix cores for every other size (any headdim,
// d_state <= 256; fp32 or bf16 storage) and its workspace (the chunks' raw
// scores at d_state <= 128; none above).
hipError_t launch_ssd_general(const SSDParams& p, bool is_bf16, hipStream_t stream);
bool ssd_general_supported(int64_t P, int64_t N);
size_t ssd_general_workspace_bytes(int64_t batch, int64_t L, int64_t N, int64_t G);
hipError_t launch_ssd_state_update(const SSDUParams& p, bool is_bf16, hipStream_t stream);
// d_state values the Mamba-2 decode kernel implements.
bool ssd_state_update_supported(int64_t N);
// dst[i] = src ? src[i] : 0 for i < n (used for zero-length sequences).
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream);

}  // namespace mssm
