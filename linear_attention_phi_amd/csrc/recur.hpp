// recur.hpp -- the token-by-token recurrence on the vector ALUs, in fp32.
//
// Used for fp32 inputs (where the fp32 tolerance rules out bf16 matrix-core
// operands) and for head dimensions of 16.  One 64-wide wave handles one
// (segment, b, h, block of 64 value columns): lane j keeps column j of S in
// registers and a 1/64 share of z, and runs
//   S <- a S + phi(k_t) v_t^T, z <- a z + phi(k_t), o_t = phi(q_t)^T S / (phi(q_t)^T z + eps)
// one token at a time ("Linear Attention: accumulating KV into a fixed-size
// state", section "State update and read as equations").  Segments are joined
// by the same prefix over segment states as the matrix-core path.
#pragma once

#include "common.hpp"
#include "scan_decode.hpp"

namespace linattn {

enum RecurMode { RECUR_STATE = 0, RECUR_CAUSAL = 1, RECUR_APPLY = 2 };

constexpr int kRecurStage = 16; // tokens staged in LDS at a time

template <typename T, int DK, bool GATED, int MODE>
__global__ __launch_bounds__(64) void recur_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                   const T *__restrict__ v, const float *__restrict__ alpha,
                                                   T *__restrict__ o, const float *__restrict__ start,
                                                   size_t start_stride_bh, size_t start_stride_seg,
                                                   const float *__restrict__ start_z, size_t start_z_stride_bh,
                                                   float *__restrict__ out_s, float *__restrict__ out_z,
                                                   size_t out_stride_bh, size_t out_stride_seg,
                                                   size_t out_z_stride_bh, float *__restrict__ gam, int N, int P,
                                                   int P_run, int seg_len, int DV, int phi_mode, float eps) {
    constexpr int ZR = (DK + 63) / 64; // z entries per lane
    __shared__ float sq[kRecurStage][DK];
    __shared__ float sk[kRecurStage][DK];
    __shared__ float sv[kRecurStage][64];
    __shared__ float sa[kRecurStage];

    const int nvb = (DV + 63) / 64;
    int bid = blockIdx.x;
    const int vb = bid % nvb;
    bid /= nvb;
    const int seg = bid % P_run, bh = bid / P_run;
    const int lane = threadIdx.x;
    const int j = vb * 64 + lane;
    const bool colok = j < DV;
    const int t_begin = seg * seg_len;
    const int t_end = MODE == RECUR_APPLY ? min(N, t_begin + seg_len) : min(N, t_begin + seg_len);

    float s[DK];
    float zo[ZR];
    {
        const float *s0 = start ? start + bh * start_stride_bh + seg * start_stride_seg : nullptr;
        const float *z0 = start_z ? start_z + bh * start_z_stride_bh + seg * start_stride_seg : nullptr;
#pragma unroll
        for (int i = 0; i < DK; ++i) s[i] = (s0 && colok) ? s0[(size_t)i * DV + j] : 0.f;
#pragma unroll
        for (int r = 0; r < ZR; ++r) {
            const int i = lane + 64 * r;
            zo[r] = (z0 && i < DK) ? z0[i] : 0.f;
        }
    }
    float gprod = 1.f;

    for (int t0 = t_begin; t0 < t_end; t0 += kRecurStage) {
        const int cnt = min(kRecurStage, t_end - t0);
        __syncthreads();
        // stage phi(q), phi(k) rows, this block's v columns and the gates
        for (int e = lane; e < kRecurStage * DK; e += 64) {
            const int t = e / DK, i = e % DK;
            const size_t row = (size_t)bh * N + t0 + t;
            float fq = 0.f, fk = 0.f;
            if (t < cnt) {
                if (MODE != RECUR_STATE) fq = phi_exact(load_elem<T>(q, row * DK + i), phi_mode);
                if (MODE != RECUR_APPLY) fk = phi_exact(load_elem<T>(k, row * DK + i), phi_mode);
            }
            sq[t][i] = fq;
            sk[t][i] = fk;
        }
        if (MODE != RECUR_APPLY) {
            for (int t = 0; t < kRecurStage; ++t)
                sv[t][lane] = (t < cnt && colok) ? load_elem<T>(v, ((size_t)bh * N + t0 + t) * DV + j) : 0.f;
            if (GATED && lane < kRecurStage) sa[lane] = lane < cnt ? alpha[(size_t)bh * N + t0 + lane] : 1.f;
        }
        __syncthreads();
        for (int t = 0; t < cnt; ++t) {
            if (MODE != RECUR_APPLY) {
                const float a = GATED ? sa[t] : 1.f;
                const float vt = sv[t][lane];
#pragma unroll
                for (int i = 0; i < DK; ++i) s[i] = GATED ? fmaf(a, s[i], sk[t][i] * vt) : fmaf(sk[t][i], vt, s[i]);
#pragma unroll
                for (int r = 0; r < ZR; ++r) {
                    const int i = lane + 64 * r;
                    if (i < DK) zo[r] = GATED ? fmaf(a, zo[r], sk[t][i]) : zo[r] + sk[t][i];
                }
                if (GATED) gprod *= a;
            }
            if (MODE != RECUR_STATE) {
                float num = 0.f, dp = 0.f;
#pragma unroll
                for (int i = 0; i < DK; ++i) num = fmaf(sq[t][i], s[i], num);
#pragma unroll
                for (int r = 0; r < ZR; ++r) {
                    const int i = lane + 64 * r;
                    if (i < DK) dp = fmaf(sq[t][i], zo[r], dp);
                }
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) dp += __shfl_xor(dp, m, 64);
                if (colok) store_elem<T>(o, ((size_t)bh * N + t0 + t) * DV + j, num / (dp + eps));
            }
        }
    }
    // states out: the segment's own state (state pass) or the final state
    // (causal pass, last segment only)
    const bool write_state = MODE == RECUR_STATE || (MODE == RECUR_CAUSAL && out_s && seg == P - 1);
    if (write_state) {
        float *ds = out_s + bh * out_stride_bh + seg * out_stride_seg;
        float *dz = out_z + bh * out_z_stride_bh + seg * out_stride_seg;
        if (colok) {
#pragma unroll
            for (int i = 0; i < DK; ++i) ds[(size_t)i * DV + j] = s[i];
        }
        if (vb == 0) {
#pragma unroll
            for (int r = 0; r < ZR; ++r) {
                const int i = lane + 64 * r;
                if (i < DK) dz[i] = zo[r];
            }
        }
        if (MODE == RECUR_STATE && GATED && vb == 0 && lane == 0) gam[(size_t)bh * P + seg] = gprod;
    }
}

} // namespace linattn
