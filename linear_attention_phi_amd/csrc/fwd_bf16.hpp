// fwd_bf16.hpp -- chunked causal linear attention on bf16 inputs, bf16 MFMA
// with fp32 accumulation and an fp32 state (gfx950, 64-wide waves).
//
// The sequence of one (batch, head) is cut into chunks of C = 64 tokens.  With
// S_0 the state before a chunk and all products taken inside the chunk, the
// recurrence S_t = S_{t-1} + phi(k_t) v_t^T, o_t = phi(q_t)^T S_t / (...)
// ("Linear Attention: accumulating KV into a fixed-size state", section "State
// update and read as equations") regroups exactly into
//   num_t = phi(q_t)^T S_0 + sum_{j<=t in chunk} (phi(q_t).phi(k_j)) v_j
//   den_t = phi(q_t)^T z_0 + sum_{j<=t in chunk}  phi(q_t).phi(k_j)
//   S_C   = S_0 + phi(K_c)^T V_c,  z_C = z_0 + colsum phi(K_c)
// i.e. the masked quadratic form of the state-space-models page (section 2) on
// the chunk plus a read of the carried summary.  With the per-token decay a_t
// every term picks up the product of the gates it has passed through.
//
// Work split of one workgroup (4 waves) over a chunk:
//   wave w owns queries 16w..16w+15: it forms the transposed score tiles
//   A^T[key][query] for key blocks 0..w, the output tile O^T[dv][query] from
//   S^T phi(Q)^T (summary read) plus V^T A^T (in-chunk part), and stores O;
//   the four waves split the Dk x Dv state update phi(K)^T V in a 2 x 2 grid
//   of accumulator tiles, and z rides along as phi(K)^T 1 on the same
//   operands.
// LDS holds the chunk's phi(K) (row-major, for the scores), phi(K)^T and V^T
// (token-contiguous, for the contractions over tokens) and a bf16 copy of
// S^T for the summary read.  The fp32 state lives in accumulator registers
// across the whole segment.
#pragma once

#include "common.hpp"

namespace linattn {

// dv index held by row m of output tile nt.  Tiles 2p and 2p+1 interleave so
// that lane (query, g) ends up with dv = 32p + 8g + 0..7 (one 16-byte store).
__device__ __forceinline__ int perm_dv(int nt, int m) {
    return 32 * (nt >> 1) + 8 * (m >> 2) + 4 * (nt & 1) + (m & 3);
}

template <int DK, int DV>
struct FwdLayout {
    static constexpr int SK = DK + 8;       // phi(K) row-major [64][DK+8]
    static constexpr int ST = kChunk + 8;   // transposed rows  [D][64+8]
    static constexpr int SS = DK + 8;       // S^T bf16         [DV][DK+8]
    static constexpr int MT = DK / 16, NT = DV / 16;
    static constexpr int MTW = MT / 2, NTW = NT / 2; // state tiles per wave (2 x 2 wave grid)
    static constexpr int KS = DK / 32;      // 32-wide k steps over Dk
};

// The fp32 state tiles one wave owns (2 x 2 wave grid over Dk x Dv), plus z
// for its Dk rows (kept on the even waves).
template <int DK, int DV>
struct StateRegs {
    f32x4 s[FwdLayout<DK, DV>::MTW][FwdLayout<DK, DV>::NTW];
    f32x4 z[FwdLayout<DK, DV>::MTW];
};

// Raw bf16 rows of one chunk held in registers between the global load and the
// LDS write: 64 tokens x D, thread -> (token group, 8-wide column group).
template <int D>
struct ChunkRows {
    static constexpr int DGS = D / 8;        // column groups of 8
    static constexpr int TPT = D / 32;       // consecutive tokens per thread
    uint4 r[TPT];
    __device__ __forceinline__ void load(const uint16_t *__restrict__ base, int rows_valid, int tid) {
        const int dg = tid % DGS, tg = tid / DGS;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int t = tg * TPT + i;
            if (t < rows_valid)
                r[i] = load_stream16(base + (size_t)t * D + dg * 8);
            else
                r[i] = make_uint4(0, 0, 0, 0);
        }
    }
};

// Write a chunk of rows to LDS transposed: dst[d][token] (row stride ST), the
// optional feature map and per-row scale applied on the way.  Rows at or past
// rows_valid are written as zeros.
template <int D, bool PHI, bool SCALE>
__device__ __forceinline__ void store_transposed(const ChunkRows<D> &cr, uint16_t *dst, int ST, int rows_valid,
                                                 int tid, int phi_mode, const float *row_scale) {
    constexpr int TPT = ChunkRows<D>::TPT, DGS = ChunkRows<D>::DGS;
    const int dg = tid % DGS, tg = tid / DGS;
    float vals[TPT][8];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const uint32_t w[4] = {cr.r[i].x, cr.r[i].y, cr.r[i].z, cr.r[i].w};
        const int t = tg * TPT + i;
        const bool ok = t < rows_valid;
        const float sc = SCALE ? row_scale[i] : 1.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo = bf_lo(w[e]), hi = bf_hi(w[e]);
            if (PHI) {
                lo = phi_fast(lo, phi_mode);
                hi = phi_fast(hi, phi_mode);
            }
            vals[i][2 * e] = ok ? lo * sc : 0.f;
            vals[i][2 * e + 1] = ok ? hi * sc : 0.f;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint16_t *p = dst + (dg * 8 + e) * ST + tg * TPT;
        if constexpr (TPT == 4) {
            uint2 u;
            u.x = pack_bf16x2(vals[0][e], vals[1][e]);
            u.y = pack_bf16x2(vals[2][e], vals[3][e]);
            *reinterpret_cast<uint2 *>(p) = u;
        } else if constexpr (TPT == 2) {
            *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(vals[0][e], vals[1][e]);
        } else {
            *p = (uint16_t)f32_to_bf16_bits(vals[0][e]);
        }
    }
}

// Write phi(K) rows row-major: dst[token][d] (row stride SK).
template <int D>
__device__ __forceinline__ void store_rows_phi(const ChunkRows<D> &cr, uint16_t *dst, int SK, int rows_valid, int tid,
                                               int phi_mode) {
    constexpr int TPT = ChunkRows<D>::TPT, DGS = ChunkRows<D>::DGS;
    const int dg = tid % DGS, tg = tid / DGS;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int t = tg * TPT + i;
        const uint32_t w[4] = {cr.r[i].x, cr.r[i].y, cr.r[i].z, cr.r[i].w};
        uint4 o;
        uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = phi_fast(bf_lo(w[e]), phi_mode), hi = phi_fast(bf_hi(w[e]), phi_mode);
            ow[e] = t < rows_valid ? pack_bf16x2(lo, hi) : 0u;
        }
        *reinterpret_cast<uint4 *>(dst + t * SK + dg * 8) = o;
    }
}

// Queries of wave w in MFMA operand layout: lane (t = l%16, g) holds
// Q[16w + t][32ks + 8g .. +7] for ks < DK/32.
template <int DK>
struct QueryRows {
    uint4 r[DK / 32];
    __device__ __forceinline__ void load(const uint16_t *__restrict__ base, int rows_valid, int w, int lane) {
        const int t = 16 * w + (lane & 15), g = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
            r[ks] = t < rows_valid ? load_stream16(base + (size_t)t * DK + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
    }
    // phi applied, rounded to bf16; rows past the end become zero.
    __device__ __forceinline__ void to_operands(bf16x8 *qa, int rows_valid, int w, int lane, int phi_mode) const {
        const bool ok = 16 * w + (lane & 15) < rows_valid;
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            const uint32_t w4[4] = {r[ks].x, r[ks].y, r[ks].z, r[ks].w};
            uint4 o;
            uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ow[e] = ok ? pack_bf16x2(phi_fast(bf_lo(w4[e]), phi_mode), phi_fast(bf_hi(w4[e]), phi_mode)) : 0u;
            qa[ks] = as_bf16x8(o);
        }
    }
};

// Per-wave gate prefix over one chunk: lane l holds the inclusive prefix
// (log2-sum of nonzero gates, count of zero gates) up to token l.  Tokens past
// the end count as gate 1.
struct ChunkGates {
    float lsum;
    int zeros;
    __device__ __forceinline__ void build(float a, bool valid) {
        const bool z = valid && gate_is_zero(a);
        lsum = (valid && !z) ? gate_log2(a) : 0.f;
        zeros = z ? 1 : 0;
        wave_inclusive_scan(lsum, zeros);
    }
    __device__ __forceinline__ float lsum_at(int t) const { return __shfl(lsum, t, 64); }
    __device__ __forceinline__ int zeros_at(int t) const { return __shfl(zeros, t, 64); }
    // this lane's token as one number (see decay_k)
    __device__ __forceinline__ float kappa() const { return lsum - kZeroShift * (float)zeros; }
    __device__ __forceinline__ float kappa_at(int t) const { return __shfl(kappa(), t, 64); }
};

// ------------------------------------------------------------------ state MFMA
// acc[mi][ni] += phi(K)^T V over the chunk for the wave's tiles; st.z[mi] +=
// phi(K)^T 1 on waves with an even index (they own distinct Dk rows).
template <int DK, int DV>
__device__ __forceinline__ void state_update(StateRegs<DK, DV> &st, const uint16_t *sKt,
                                             const uint16_t *sVt, int w, int lane) {
    using L = FwdLayout<DK, DV>;
    const int l16 = lane & 15, g = lane >> 4;
    const int mt0 = (w >> 1) * L::MTW, nt0 = (w & 1) * L::NTW;
    bf16x8 ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
#pragma unroll
    for (int ks = 0; ks < kChunk / 32; ++ks) {
        bf16x8 a[L::MTW], b[L::NTW];
#pragma unroll
        for (int mi = 0; mi < L::MTW; ++mi)
            a[mi] = *reinterpret_cast<const bf16x8 *>(sKt + (16 * (mt0 + mi) + l16) * L::ST + 32 * ks + 8 * g);
#pragma unroll
        for (int ni = 0; ni < L::NTW; ++ni)
            b[ni] = *reinterpret_cast<const bf16x8 *>(sVt + (16 * (nt0 + ni) + l16) * L::ST + 32 * ks + 8 * g);
#pragma unroll
        for (int mi = 0; mi < L::MTW; ++mi) {
#pragma unroll
            for (int ni = 0; ni < L::NTW; ++ni) st.s[mi][ni] = mfma16x16x32(a[mi], b[ni], st.s[mi][ni]);
        }
        if ((w & 1) == 0) {
#pragma unroll
            for (int mi = 0; mi < L::MTW; ++mi) st.z[mi] = mfma16x16x32(a[mi], ones, st.z[mi]);
        }
    }
}

// Load / store the fp32 state of the wave's tiles from / to global memory
// laid out [Dk][Dv] then z[Dk].  src == nullptr loads zeros.
template <int DK, int DV>
__device__ __forceinline__ void state_load(StateRegs<DK, DV> &st, const float *s, const float *z,
                                           int w, int lane) {
    using L = FwdLayout<DK, DV>;
    const int l16 = lane & 15, g = lane >> 4;
    const int mt0 = (w >> 1) * L::MTW, nt0 = (w & 1) * L::NTW;
#pragma unroll
    for (int mi = 0; mi < L::MTW; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dk = 16 * (mt0 + mi) + 4 * g + i;
#pragma unroll
            for (int ni = 0; ni < L::NTW; ++ni)
                st.s[mi][ni][i] = s ? s[dk * DV + 16 * (nt0 + ni) + l16] : 0.f;
            st.z[mi][i] = z ? z[dk] : 0.f;
        }
    }
}

template <int DK, int DV>
__device__ __forceinline__ void state_store(const StateRegs<DK, DV> &st, float *s, float *z, int w,
                                            int lane) {
    using L = FwdLayout<DK, DV>;
    const int l16 = lane & 15, g = lane >> 4;
    const int mt0 = (w >> 1) * L::MTW, nt0 = (w & 1) * L::NTW;
#pragma unroll
    for (int mi = 0; mi < L::MTW; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dk = 16 * (mt0 + mi) + 4 * g + i;
#pragma unroll
            for (int ni = 0; ni < L::NTW; ++ni) s[dk * DV + 16 * (nt0 + ni) + l16] = st.s[mi][ni][i];
            if ((w & 1) == 0 && l16 == 0) z[dk] = st.z[mi][i];
        }
    }
}

// bf16 copy of S^T ([dv][dk]) and fp32 z into LDS for the summary read.
template <int DK, int DV>
__device__ __forceinline__ void state_to_lds(const StateRegs<DK, DV> &st, uint16_t *sSt, float *sZ,
                                             int w, int lane) {
    using L = FwdLayout<DK, DV>;
    const int l16 = lane & 15, g = lane >> 4;
    const int mt0 = (w >> 1) * L::MTW, nt0 = (w & 1) * L::NTW;
#pragma unroll
    for (int mi = 0; mi < L::MTW; ++mi) {
#pragma unroll
        for (int ni = 0; ni < L::NTW; ++ni) {
            uint2 u;
            u.x = pack_bf16x2(st.s[mi][ni][0], st.s[mi][ni][1]);
            u.y = pack_bf16x2(st.s[mi][ni][2], st.s[mi][ni][3]);
            *reinterpret_cast<uint2 *>(sSt + (16 * (nt0 + ni) + l16) * L::SS + 16 * (mt0 + mi) + 4 * g) = u;
        }
        if ((w & 1) == 0 && l16 == 0)
            *reinterpret_cast<float4 *>(sZ + 16 * (mt0 + mi) + 4 * g) =
                make_float4(st.z[mi][0], st.z[mi][1], st.z[mi][2], st.z[mi][3]);
    }
}

template <int DK, int DV>
__device__ __forceinline__ void state_scale(StateRegs<DK, DV> &st, float d) {
    using L = FwdLayout<DK, DV>;
#pragma unroll
    for (int mi = 0; mi < L::MTW; ++mi) {
#pragma unroll
        for (int ni = 0; ni < L::NTW; ++ni) st.s[mi][ni] *= d;
        st.z[mi] *= d;
    }
}

// Per-row decay from each of this thread's chunk rows to the chunk end.
template <int D>
__device__ __forceinline__ void rows_to_end_decay(const ChunkGates &cg, int last, int tid, float *out) {
    constexpr int TPT = ChunkRows<D>::TPT, DGS = ChunkRows<D>::DGS;
    const int tg = tid / DGS;
    const float le = cg.lsum_at(last);
    const int ze = cg.zeros_at(last);
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int t = tg * TPT + i;
        out[i] = decay_between(le, ze, cg.lsum_at(t), cg.zeros_at(t));
    }
}

// ====================================================================== kernels
// Both chunk kernels keep two chunks of loads in flight: the registers of
// buffer c % 2 are staged into LDS for chunk c and immediately reloaded with
// chunk c + 2, so the loads of two chunks overlap the compute of one.

// Segment-state pass: for segment p of (b, h), the state the segment adds when
// started from zero: dS = sum phi(k_j) v_j^T (decayed to the segment end when
// gated), dz likewise, and the segment's total gate product.
// Grid: one workgroup per (segment, bh) with segment index fastest; P_run
// segments are computed, their results stored at stride P.
template <int DK, int DV, bool GATED>
__global__ __launch_bounds__(kThreads, 2) void seg_state_bf16(const uint16_t *__restrict__ k,
                                                              const uint16_t *__restrict__ v,
                                                              const float *__restrict__ alpha, float *__restrict__ ws,
                                                              float *__restrict__ gam, int N, int P, int P_run,
                                                              int seg_len, int phi_mode) {
    using L = FwdLayout<DK, DV>;
    __shared__ __attribute__((aligned(16))) uint16_t sKt[DK * L::ST];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[DV * L::ST];

    const int seg = blockIdx.x % P_run, bh = blockIdx.x / P_run;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int t_begin = seg * seg_len;
    const int t_end = min(N, t_begin + seg_len);
    const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
    const uint16_t *kb = k + ((size_t)bh * N + t_begin) * DK;
    const uint16_t *vb = v + ((size_t)bh * N + t_begin) * DV;
    const float *ab = GATED ? alpha + (size_t)bh * N + t_begin : nullptr;

    StateRegs<DK, DV> sr;
    state_load<DK, DV>(sr, nullptr, nullptr, w, lane);
    float seg_lsum = 0.f;
    int seg_zeros = 0;

    struct Buf {
        ChunkRows<DK> kr;
        ChunkRows<DV> vr;
        float a;
    };
    auto rows_in = [&](int c) { return min(kChunk, t_end - t_begin - c * kChunk); };
    auto issue = [&](Buf &b, int c) {
        const int nv = rows_in(c);
        b.kr.load(kb + (size_t)c * kChunk * DK, nv, tid);
        b.vr.load(vb + (size_t)c * kChunk * DV, nv, tid);
        if (GATED) b.a = lane < nv ? ab[c * kChunk + lane] : 1.f;
    };
    auto step = [&](Buf &b, int c) {
        const int valid = rows_in(c);
        float dC = 1.f;
        if (GATED) {
            ChunkGates cg;
            cg.build(b.a, lane < valid);
            float rs[ChunkRows<DK>::TPT];
            rows_to_end_decay<DK>(cg, valid - 1, tid, rs);
            store_transposed<DK, true, true>(b.kr, sKt, L::ST, valid, tid, phi_mode, rs);
            const float le = cg.lsum_at(valid - 1);
            const int ze = cg.zeros_at(valid - 1);
            dC = decay_between(le, ze, 0.f, 0);
            seg_lsum += le;
            seg_zeros += ze;
        } else {
            store_transposed<DK, true, false>(b.kr, sKt, L::ST, valid, tid, phi_mode, nullptr);
        }
        store_transposed<DV, false, false>(b.vr, sVt, L::ST, valid, tid, phi_mode, nullptr);
        if (c + 2 < nch) issue(b, c + 2);
        __syncthreads();
        if (GATED) state_scale<DK, DV>(sr, dC);
        state_update<DK, DV>(sr, sKt, sVt, w, lane);
        __syncthreads();
    };
    Buf b0, b1;
    issue(b0, 0);
    if (nch > 1) issue(b1, 1);
    for (int c = 0; c < nch; c += 2) {
        step(b0, c);
        if (c + 1 < nch) step(b1, c + 1);
    }
    float *dst = ws + ((size_t)bh * P + seg) * (size_t)(DK * DV + DK);
    state_store<DK, DV>(sr, dst, dst + DK * DV, w, lane);
    if (GATED && tid == 0) gam[(size_t)bh * P + seg] = seg_zeros > 0 ? 0.f : __builtin_amdgcn_exp2f(seg_lsum);
}

// Causal output pass: segment p of (b, h) starts from the state before it
// (start_s/start_z, or zeros when null), runs the chunked form over its
// tokens, writes O, and the last segment writes the final state.
template <int DK, int DV, bool GATED>
__global__ __launch_bounds__(kThreads, 1) void fwd_out_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, uint16_t *__restrict__ o, const float *__restrict__ start, size_t start_stride_bh,
    size_t start_stride_seg, const float *__restrict__ start_z, size_t start_z_stride_bh, float *__restrict__ s_final,
    float *__restrict__ z_final, int N, int P, int seg_len, int phi_mode, float eps) {
    using L = FwdLayout<DK, DV>;
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * L::SK];
    __shared__ __attribute__((aligned(16))) uint16_t sKt[DK * L::ST];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[DV * L::ST];
    __shared__ __attribute__((aligned(16))) uint16_t sSt[DV * L::SS];
    __shared__ __attribute__((aligned(16))) float sZ[DK];

    const int seg = blockIdx.x % P, bh = blockIdx.x / P;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int t_begin = seg * seg_len;
    const int t_end = min(N, t_begin + seg_len);
    const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
    const size_t row0 = (size_t)bh * N + t_begin;
    const uint16_t *qb = q + row0 * DK;
    const uint16_t *kb = k + row0 * DK;
    const uint16_t *vb = v + row0 * DV;
    uint16_t *ob = o + row0 * DV;
    const float *ab = GATED ? alpha + row0 : nullptr;

    StateRegs<DK, DV> sr;
    {
        const float *s0 = start ? start + bh * start_stride_bh + seg * start_stride_seg : nullptr;
        const float *z0 = start_z ? start_z + bh * start_z_stride_bh + seg * start_stride_seg : nullptr;
        state_load<DK, DV>(sr, s0, z0, w, lane);
    }
    state_to_lds<DK, DV>(sr, sSt, sZ, w, lane);

    struct Buf {
        ChunkRows<DK> kr;
        ChunkRows<DV> vr;
        QueryRows<DK> qr;
        float a;
    };
    auto rows_in = [&](int c) { return min(kChunk, t_end - t_begin - c * kChunk); };
    auto issue = [&](Buf &b, int c) {
        const int nv = rows_in(c);
        b.kr.load(kb + (size_t)c * kChunk * DK, nv, tid);
        b.vr.load(vb + (size_t)c * kChunk * DV, nv, tid);
        b.qr.load(qb + (size_t)c * kChunk * DK, nv, w, lane);
        if (GATED) b.a = lane < nv ? ab[c * kChunk + lane] : 1.f;
    };
    auto step = [&](Buf &b, int c) {
        const int valid = rows_in(c);
        // ---- stage the chunk: phi(K) both ways, V^T, phi(Q) operands, gates
        bf16x8 qa[L::KS];
        b.qr.to_operands(qa, valid, w, lane, phi_mode);
        ChunkGates cg;
        float dC = 1.f;
        if (GATED) {
            cg.build(b.a, lane < valid);
            float rs[ChunkRows<DK>::TPT];
            rows_to_end_decay<DK>(cg, valid - 1, tid, rs);
            store_transposed<DK, true, true>(b.kr, sKt, L::ST, valid, tid, phi_mode, rs);
            dC = decay_between(cg.lsum_at(valid - 1), cg.zeros_at(valid - 1), 0.f, 0);
        } else {
            store_transposed<DK, true, false>(b.kr, sKt, L::ST, valid, tid, phi_mode, nullptr);
        }
        store_rows_phi<DK>(b.kr, sK, L::SK, valid, tid, phi_mode);
        store_transposed<DV, false, false>(b.vr, sVt, L::ST, valid, tid, phi_mode, nullptr);
        // ---- refill this buffer with the chunk after next
        if (c + 2 < nch) issue(b, c + 2);
        __syncthreads();

        // ---- scores A^T[key][query] for key blocks 0..w
        f32x4 sc[4];
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
            sc[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (kb4 <= w) {
#pragma unroll
                for (int ks = 0; ks < L::KS; ++ks) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8 *>(sK + (16 * kb4 + l16) * L::SK + 32 * ks + 8 * g);
                    sc[kb4] = mfma16x16x32(a, qa[ks], sc[kb4]);
                }
            }
        }
        const int tq = 16 * w + l16; // this lane's query within the chunk
        float lq = 0.f;
        int zq = 0;
        if (GATED) {
            lq = cg.lsum_at(tq);
            zq = cg.zeros_at(tq);
        }
        float den = 0.f;
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tk = 16 * kb4 + 4 * g + i;
                float s = sc[kb4][i];
                if (tk > tq) s = 0.f;
                if (GATED) s *= decay_between(lq, zq, cg.lsum_at(tk), cg.zeros_at(tk));
                sc[kb4][i] = s;
                den += s;
            }
        }
        den = sum_over_groups(den);

        // ---- summary read: O^T = S^T phi(Q)^T, den += phi(q).z
        f32x4 oacc[L::NT];
#pragma unroll
        for (int nt = 0; nt < L::NT; ++nt) {
            oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int dv = perm_dv(nt, l16);
#pragma unroll
            for (int ks = 0; ks < L::KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sSt + dv * L::SS + 32 * ks + 8 * g);
                oacc[nt] = mfma16x16x32(a, qa[ks], oacc[nt]);
            }
        }
        float dz = 0.f;
#pragma unroll
        for (int ks = 0; ks < L::KS; ++ks) {
            const float4 z0 = *reinterpret_cast<const float4 *>(sZ + 32 * ks + 8 * g);
            const float4 z1 = *reinterpret_cast<const float4 *>(sZ + 32 * ks + 8 * g + 4);
            const uint4 u = as_u4(qa[ks]);
            dz += bf_lo(u.x) * z0.x + bf_hi(u.x) * z0.y + bf_lo(u.y) * z0.z + bf_hi(u.y) * z0.w;
            dz += bf_lo(u.z) * z1.x + bf_hi(u.z) * z1.y + bf_lo(u.w) * z1.z + bf_hi(u.w) * z1.w;
        }
        dz = sum_over_groups(dz);
        if (GATED) {
            const float dq = decay_between(lq, zq, 0.f, 0);
            dz *= dq;
#pragma unroll
            for (int nt = 0; nt < L::NT; ++nt) oacc[nt] *= dq;
        }
        den += dz;

        // ---- in-chunk part: O^T += V^T A^T over key blocks 0..w
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            if (2 * s2 <= w) {
                uint4 bu;
                bu.x = pack_bf16x2(sc[2 * s2][0], sc[2 * s2][1]);
                bu.y = pack_bf16x2(sc[2 * s2][2], sc[2 * s2][3]);
                bu.z = pack_bf16x2(sc[2 * s2 + 1][0], sc[2 * s2 + 1][1]);
                bu.w = pack_bf16x2(sc[2 * s2 + 1][2], sc[2 * s2 + 1][3]);
                const bf16x8 bop = as_bf16x8(bu);
#pragma unroll
                for (int nt = 0; nt < L::NT; ++nt) {
                    const int dv = perm_dv(nt, l16);
                    const uint2 lo = *reinterpret_cast<const uint2 *>(sVt + dv * L::ST + 32 * s2 + 4 * g);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(sVt + dv * L::ST + 32 * s2 + 16 + 4 * g);
                    oacc[nt] = mfma16x16x32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), bop, oacc[nt]);
                }
            }
        }

        // ---- normalize and store this wave's 16 rows
        if (tq < valid) {
            const float inv = __builtin_amdgcn_rcpf(den + eps); // 1 ulp; the result is rounded to bf16
            uint16_t *orow = ob + ((size_t)c * kChunk + tq) * DV;
#pragma unroll
            for (int p = 0; p < DV / 32; ++p) {
                uint4 u;
                u.x = pack_bf16x2(oacc[2 * p][0] * inv, oacc[2 * p][1] * inv);
                u.y = pack_bf16x2(oacc[2 * p][2] * inv, oacc[2 * p][3] * inv);
                u.z = pack_bf16x2(oacc[2 * p + 1][0] * inv, oacc[2 * p + 1][1] * inv);
                u.w = pack_bf16x2(oacc[2 * p + 1][2] * inv, oacc[2 * p + 1][3] * inv);
                *reinterpret_cast<uint4 *>(orow + 32 * p + 8 * g) = u;
            }
        }

        // ---- carry the state across the chunk
        if (GATED) state_scale<DK, DV>(sr, dC);
        state_update<DK, DV>(sr, sKt, sVt, w, lane);
        __syncthreads();
        if (c + 1 < nch) state_to_lds<DK, DV>(sr, sSt, sZ, w, lane);
    };

    Buf b0, b1;
    issue(b0, 0);
    if (nch > 1) issue(b1, 1);
    for (int c = 0; c < nch; c += 2) {
        step(b0, c);
        if (c + 1 < nch) step(b1, c + 1);
    }
    if (s_final && seg == P - 1)
        state_store<DK, DV>(sr, s_final + (size_t)bh * DK * DV, z_final + (size_t)bh * DK, w, lane);
}

// Non-causal read: every query of (b, h) reads the one global state.
// Grid: one workgroup per (block of chunks, bh), block index fastest.
template <int DK, int DV, int PHI>
__global__ __launch_bounds__(kThreads, 2) void noncausal_apply_bf16(const uint16_t *__restrict__ q,
                                                                    uint16_t *__restrict__ o,
                                                                    const float *__restrict__ total, int N,
                                                                    int blocks_per_bh, int chunks_per_block,
                                                                    float eps) {
    constexpr int phi_mode = PHI; // 0: elu + 1, 1: identity (compile-time)
    using L = FwdLayout<DK, DV>;
    __shared__ __attribute__((aligned(16))) uint16_t sSt[DV * L::SS];
    __shared__ __attribute__((aligned(16))) float sZ[DK];
    const int blk = blockIdx.x % blocks_per_bh, bh = blockIdx.x / blocks_per_bh;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    {
        StateRegs<DK, DV> sr;
        const float *s0 = total + (size_t)bh * (DK * DV + DK);
        state_load<DK, DV>(sr, s0, s0 + DK * DV, w, lane);
        state_to_lds<DK, DV>(sr, sSt, sZ, w, lane);
    }
    __syncthreads();
    const int c0 = blk * chunks_per_block;
    const int c1 = min((N + kChunk - 1) / kChunk, c0 + chunks_per_block);
    const int t = 16 * w + l16; // this lane's query row within a chunk
    const uint16_t *qh = q + (size_t)bh * N * DK;
    // The next chunk's Q rows are loaded while this one is computed.  Loads and
    // stores are bounded to the chunk's valid rows (rows past the end read as
    // zero, and their outputs are dropped by the store's bounds, with no branch
    // around it: the compiler then counts every store, and the wait for the next
    // chunk's loads does not cover them); past the block's last chunk the range
    // is empty, so the loop needs no branch around the loads either.
    auto rows_in = [&](int c) { return c < c1 ? min(kChunk, N - c * kChunk) : 0; };
    auto qload = [&](uint4 (&r)[L::KS], int c) {
        const rsrc_t rs = chunk_rsrc(qh + (size_t)c * kChunk * DK, rows_in(c) * DK * 2);
#pragma unroll
        for (int ks = 0; ks < L::KS; ++ks) r[ks] = buffer_load16<true>(rs, (t * DK + 32 * ks + 8 * g) * 2);
    };
    auto process = [&](const uint4 (&r)[L::KS], int c) {
        const int valid = rows_in(c);
        bf16x8 qa[L::KS];
#pragma unroll
        for (int ks = 0; ks < L::KS; ++ks) {
            const uint32_t w4[4] = {r[ks].x, r[ks].y, r[ks].z, r[ks].w};
            uint4 o4;
            uint32_t *ow = reinterpret_cast<uint32_t *>(&o4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ow[e] = pack_bf16x2(phi_fast(bf_lo(w4[e]), phi_mode), phi_fast(bf_hi(w4[e]), phi_mode));
            qa[ks] = as_bf16x8(o4);
        }
        f32x4 oacc[L::NT];
#pragma unroll
        for (int nt = 0; nt < L::NT; ++nt) {
            oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int dv = perm_dv(nt, l16);
#pragma unroll
            for (int ks = 0; ks < L::KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sSt + dv * L::SS + 32 * ks + 8 * g);
                oacc[nt] = mfma16x16x32(a, qa[ks], oacc[nt]);
            }
        }
        float den = 0.f;
#pragma unroll
        for (int ks = 0; ks < L::KS; ++ks) {
            const float4 z0 = *reinterpret_cast<const float4 *>(sZ + 32 * ks + 8 * g);
            const float4 z1 = *reinterpret_cast<const float4 *>(sZ + 32 * ks + 8 * g + 4);
            const uint4 u = as_u4(qa[ks]);
            den += bf_lo(u.x) * z0.x + bf_hi(u.x) * z0.y + bf_lo(u.y) * z0.z + bf_hi(u.y) * z0.w;
            den += bf_lo(u.z) * z1.x + bf_hi(u.z) * z1.y + bf_lo(u.w) * z1.z + bf_hi(u.w) * z1.w;
        }
        den = sum_over_groups(den);
        {
            const float inv = __builtin_amdgcn_rcpf(den + eps); // 1 ulp; the result is rounded to bf16
            const rsrc_t ro = chunk_rsrc(o + ((size_t)bh * N + (size_t)c * kChunk) * DV, valid * DV * 2);
#pragma unroll
            for (int p = 0; p < DV / 32; ++p) {
                uint4 u;
                u.x = pack_bf16x2(oacc[2 * p][0] * inv, oacc[2 * p][1] * inv);
                u.y = pack_bf16x2(oacc[2 * p][2] * inv, oacc[2 * p][3] * inv);
                u.z = pack_bf16x2(oacc[2 * p + 1][0] * inv, oacc[2 * p + 1][1] * inv);
                u.w = pack_bf16x2(oacc[2 * p + 1][2] * inv, oacc[2 * p + 1][3] * inv);
                buffer_store16(u, ro, (t * DV + 32 * p + 8 * g) * 2);
            }
        }
    };
    uint4 r0[L::KS], r1[L::KS];
    qload(r0, c0);
    int c = c0;
    for (; c + 1 < c1; c += 2) {
        qload(r1, c + 1);
        process(r0, c);
        qload(r0, c + 2);
        process(r1, c + 1);
    }
    if (c < c1) process(r0, c);
}

} // namespace linattn
