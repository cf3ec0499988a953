// bwd8_bf16.hpp -- backward of the chunked causal linear attention (ungated),
// eight waves per workgroup, head dims Dk, Dv in {64, 128}, bf16 in and out,
// fp32 state.
//
// With dY_t = dO_t / den_t and dd_t = -(dO_t . o_t) / den_t (den_t = phi(q_t).z_t
// + eps), the gradients of the forward of fwd8_bf16.hpp are, with S_t, z_t
// the forward state after token t and
// R_t = sum_{u >= t} phi(q_u) dY_u^T, r_t = sum_{u >= t} dd_u phi(q_u):
//   dphi(q_t) = S_t dY_t + dd_t z_t
//   dphi(k_t) = R_t v_t + r_t
//   dv_t      = R_t^T phi(k_t)
// and dq = dphi(q) phi'(q), dk = dphi(k) phi'(k), where phi'(x) = min(1, phi(x))
// for elu + 1 (1 on x >= 0 where phi(x) = x + 1 >= 1, exp(x) = phi(x) < 1 below)
// and 1 for the identity map.  Chunked like the forward (64 tokens):
//   dphi(Q)_c = dY_c S_{c-1}^T + dd_c z_{c-1}^T + tril(dY_c V_c^T + dd_c 1^T) phi(K)_c
//   dphi(K)_c = V_c R_{c+1}^T + 1 r_{c+1}^T + triu(V_c dY_c^T + 1 dd_c^T) phi(Q)_c
//   dV_c      = phi(K)_c R_{c+1} + triu(phi(K)_c phi(Q)_c^T) dY_c
// (tril / triu over (query, key) with the diagonal included).  Passes: the
// state pass gives the forward state at segment starts (or the training
// forward's saved cells serve); bwd_dq8_bf16 runs each segment forward in
// time, writes dd, and sums R and r over the segment from the phi(Q), dY and
// dd it has staged (for a suffix over segments);
// bwd_dkv8_bf16 runs each segment backward in time.  dY is dO over the
// forward's saved denominator, rounded to bf16 once; every pass uses that
// same dY.
//
// Precision of dq.  dphi(q_t) = sum_j phi(k_j) (v_j - o_t) . dY_t satisfies
// phi(q_t) . dphi(q_t) = 0 up to eps: for elu + 1 its part along the all-ones
// direction cancels, and for inputs of small spread the result is far smaller
// than its terms.  A bf16 phi(k) = 1 + elu(k) keeps elu(k) only to 2^-8
// absolute, and an o rounded anywhere on its way (a bf16 score or output in
// the forward) moves the cancelling terms by 2^-9 of their size; either alone
// leaves percent-level errors in dq.  The dq pass therefore
//  * writes phi = 1 + elu and carries the constant part in fp32:
//      S_t = E_t + 1 Vbar_t^T,  z_t = zeta_t + n_t 1,
//      dphi(q_t) = E_t dY_t + dd_t zeta_t + (Vbar_t . dY_t + n_t dd_t) 1,
//    with E = sum elu(k) v^T and zeta = sum elu(k) (bf16 operands of full
//    relative precision), Vbar = sum v and n the token count (fp32), and the
//    in-chunk sums over keys taken from the fp32 accumulators;
//  * forms dd from its own state rather than from the forward's o:
//      dd_t = -phi(q_t) . (S_t dY_t) / (phi(q_t) . z_t + eps),
//    the same S_t, z_t that the gradient uses, so that the cancellation is
//    exact in the arithmetic the pass carries out.  dd goes to the workspace
//    for the dK, dV pass, and into the reverse sums.
#pragma once

#include "fwd8_bf16.hpp"

namespace linattn {

// The lane index, hidden from loop-invariant code motion: the per-lane LDS
// addresses of a chunk's many operand reads are then recomputed inside the
// chunk loop (a few VALU ops beside the MFMAs) instead of all being hoisted
// out of it and held in registers for the whole loop.
__device__ __forceinline__ int lane_in_loop(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}

// 1 / den for dY = dO / den; rows past the end (den read as 0) get 0.  The
// hardware reciprocal (1 ulp) in place of a correctly rounded division: dY is
// rounded to bf16 next, and every pass forms it with this same function.
__device__ __forceinline__ float dy_inv(float den) { return den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f; }

// Eight elements of dY = dO / den, rounded to bf16 as every pass uses them.
__device__ __forceinline__ uint4 dy_pack8(uint4 g, float inv) {
    return make_uint4(pack_bf16x2(bf_lo(g.x) * inv, bf_hi(g.x) * inv), pack_bf16x2(bf_lo(g.y) * inv, bf_hi(g.y) * inv),
                      pack_bf16x2(bf_lo(g.z) * inv, bf_hi(g.z) * inv), pack_bf16x2(bf_lo(g.w) * inv, bf_hi(g.w) * inv));
}

// Per-thread loads of one chunk for the backward: Q, K, V, dO rows, and the
// saved denominators (and, with DD, dd) of this thread's dO rows.
template <int DK, int DV, bool DD = true>
struct BwdBuf {
    Units<DK> q, k;
    Units<DV> v, g;
    float den[Units<DV>::N], dd[Units<DV>::N];
    __device__ __forceinline__ void load(const uint16_t *qb, const uint16_t *kb, const uint16_t *vb, const uint16_t *gb,
                                         const float *db, const float *ddb, int rows_valid, int tid) {
        q.load(qb, rows_valid, tid);
        k.load(kb, rows_valid, tid);
        v.load(vb, rows_valid, tid);
        g.load(gb, rows_valid, tid);
        const rsrc_t rs = chunk_rsrc(db, rows_valid * 4);
#pragma unroll
        for (int i = 0; i < Units<DV>::N; ++i) den[i] = buffer_load_f32(rs, Units<DV>::row_of(tid, i) * 4);
        if constexpr (DD) {
            const rsrc_t rd = chunk_rsrc(ddb, rows_valid * 4);
#pragma unroll
            for (int i = 0; i < Units<DV>::N; ++i) dd[i] = buffer_load_f32(rd, Units<DV>::row_of(tid, i) * 4);
        }
    }
};

// Stage dY = dO / den (bf16, Tile<DV>) and, when sDD is given, dd (fp32 per
// row).  Rows past the end read den = 0 and dd = 0 and get dY = 0.
template <int DV>
__device__ __forceinline__ void stage_dy(const Units<DV> &g, const float (&den)[Units<DV>::N],
                                         const float (&dd)[Units<DV>::N], uint16_t *sDY, float *sDD, int tid) {
#pragma unroll
    for (int i = 0; i < Units<DV>::N; ++i) {
        const int row = Units<DV>::row_of(tid, i), col = Units<DV>::col_of(tid, i);
        *reinterpret_cast<uint4 *>(sDY + Tile<DV>::off(row, col)) = dy_pack8(g.r[i], dy_inv(den[i]));
        if (sDD && col == 0) sDD[row] = dd[i];
    }
}

// The dQ pass's staging: phi(Q) in bf16 (the values every later use of phi(q)
// reads, so that the pass's dd stays consistent with its own arithmetic), the
// row sums of those bf16 values in fp32 (sum over the DK / 8 consecutive lanes
// of a row, into sSq[row]), the features KF of K, and V as is.
template <int DK, int DV, int PHI, int KF, bool DD>
__device__ __forceinline__ void stage_dq(const BwdBuf<DK, DV, DD> &b, uint16_t *sQ, uint16_t *sK, uint16_t *sV,
                                         float *sSq, int tid) {
    constexpr int CG = Units<DK>::CG;
#pragma unroll
    for (int i = 0; i < Units<DK>::N; ++i) {
        const int row = Units<DK>::row_of(tid, i), col = Units<DK>::col_of(tid, i);
        const uint4 f = phi_pack8(b.q.r[i], PHI);
        *reinterpret_cast<uint4 *>(sQ + Tile<DK>::off(row, col)) = f;
        const uint32_t fw[4] = {f.x, f.y, f.z, f.w};
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) x += bf_lo(fw[e]) + bf_hi(fw[e]);
        if constexpr (CG == 16) {
            x = row16_sum(x);
        } else {
#pragma unroll
            for (int m = 1; m < CG; m <<= 1) x += __shfl_xor(x, m, 64);
        }
        if (col == 0) sSq[row] = x;
        *reinterpret_cast<uint4 *>(sK + Tile<DK>::off(row, col)) = phi_pack8(b.k.r[i], KF);
    }
#pragma unroll
    for (int i = 0; i < Units<DV>::N; ++i)
        *reinterpret_cast<uint4 *>(sV + Tile<DV>::off(Units<DV>::row_of(tid, i), Units<DV>::col_of(tid, i))) =
            b.v.r[i];
}

// The staged Q and K rows into their tiles through feature maps QF / KF
// (phi_fast modes), and V as is.
template <int F>
__device__ __forceinline__ uint4 feat8(uint4 raw) {
    return phi_pack8(raw, F);
}
template <int DK, int DV, int QF, int KF, bool DD>
__device__ __forceinline__ void stage_qkv(const BwdBuf<DK, DV, DD> &b, uint16_t *sQ, uint16_t *sK, uint16_t *sV,
                                          int tid) {
#pragma unroll
    for (int i = 0; i < Units<DK>::N; ++i) {
        const int row = Units<DK>::row_of(tid, i), col = Units<DK>::col_of(tid, i);
        *reinterpret_cast<uint4 *>(sQ + Tile<DK>::off(row, col)) = feat8<QF>(b.q.r[i]);
        *reinterpret_cast<uint4 *>(sK + Tile<DK>::off(row, col)) = feat8<KF>(b.k.r[i]);
    }
#pragma unroll
    for (int i = 0; i < Units<DV>::N; ++i)
        *reinterpret_cast<uint4 *>(sV + Tile<DV>::off(Units<DV>::row_of(tid, i), Units<DV>::col_of(tid, i))) =
            b.v.r[i];
}

// A operand rows m -> row index perm_dv(nt, m) (k along the row) from a TileS
// [rows][Dv] tile: two 8-byte reads per lane.
template <int DV>
__device__ __forceinline__ bf16x8 tiles_row_operand(const uint16_t *t, int row, int col) {
    const uint2 lo = *reinterpret_cast<const uint2 *>(t + TileS<DV>::off(row, col));
    const uint2 hi = *reinterpret_cast<const uint2 *>(t + TileS<DV>::off(row, col + 4));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// phi'(x) for elu + 1 (1 for the identity map): 1 on x >= 0, exp(x) below,
// read from phi(x) = exp(x) < 1 there (kScalePhi).
constexpr int kScaleNone = 0, kScalePhi = 1;
template <int PHI, int MODE>
__device__ __forceinline__ float dphi_of(float f) {
    if (PHI || MODE == kScaleNone) return 1.f;
    return fminf(1.f, f);
}

// Store 16 rows x (2 * NTW) permuted tiles of a gradient, scaled by phi'
// (from the staged tile given, per MODE): lane (g, l16) holds, for tile pair
// p, the 8 consecutive columns 32 p + 8 g .. + 7 of row l16.  out: the
// chunk's output rows (row tile_row of them is this lane's), bounded to the
// chunk's valid rows (stores past them are dropped).
template <int D, int NTW, int MODE, int PHI>
__device__ __forceinline__ void store_grad_rows(const f32x4 (&acc)[NTW], int nt0, const uint16_t *phi_tile,
                                                int tile_row, rsrc_t out, int g) {
    constexpr bool SCALE = MODE != kScaleNone && !PHI;
#pragma unroll
    for (int pp = 0; pp < NTW / 2; ++pp) {
        const int p = (nt0 >> 1) + pp;
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = acc[2 * pp][i];
            x[4 + i] = acc[2 * pp + 1][i];
        }
        if (SCALE) {
            const uint4 f = *reinterpret_cast<const uint4 *>(phi_tile + Tile<D>::off(tile_row, 32 * p + 8 * g));
            const uint32_t fw[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] *= dphi_of<PHI, MODE>(bf_lo(fw[e]));
                x[2 * e + 1] *= dphi_of<PHI, MODE>(bf_hi(fw[e]));
            }
        }
        uint4 u;
        u.x = pack_bf16x2(x[0], x[1]);
        u.y = pack_bf16x2(x[2], x[3]);
        u.z = pack_bf16x2(x[4], x[5]);
        u.w = pack_bf16x2(x[6], x[7]);
        buffer_store16(u, out, (tile_row * D + 32 * p + 8 * g) * 2);
    }
}

// Eight dd values of tokens 32 ks + 8 G .. + 7 (the state update's operand
// order for lane group G) as a bf16 MFMA operand.
__device__ __forceinline__ bf16x8 dd_operand(const float *sDD, int ks, int G) {
    const float4 a = *reinterpret_cast<const float4 *>(sDD + 32 * ks + 8 * G);
    const float4 b = *reinterpret_cast<const float4 *>(sDD + 32 * ks + 8 * G + 4);
    return as_bf16x8(make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                                pack_bf16x2(b.z, b.w)));
}

// The state update of state8_update with ones for z, which also sums the V
// rows over the chunk (the column sums that carry Vbar) on the matrix cores:
// V^T times a ones operand gives each column's sum in every output column.
// The waves of the first key-dim block (which between them hold every
// value-dim tile) do the extra products; lane 16 g of such a wave then holds
// the sums of columns 16 (nt0 + ni) + 4 g + i and writes them to vd[Dv].
template <int DK, int DV>
__device__ __forceinline__ void state8_update_vcol(State8<DK, DV> &st, const uint16_t *kt, const uint16_t *vt, int w,
                                                   int lane, bf16x8 ones, float *vd) {
    using S = State8<DK, DV>;
    const int G = lane >> 4, q = lane & 3, mt0 = (w >> 2) * S::MTW, nt0 = (w & 3) * S::NTW;
    const int zmi = S::zmi(w);
    const bool vcol = mt0 == 0;
    f32x4 vc[S::NTW];
#pragma unroll
    for (int ni = 0; ni < S::NTW; ++ni) vc[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kChunk / 32; ++ks) {
        const int klo = 32 * ks + 8 * G, khi = klo + 4;
        bf16x8 a[S::MTW], b[S::NTW];
#pragma unroll
        for (int mi = 0; mi < S::MTW; ++mi) a[mi] = tr_operand<DK>(kt, klo, khi, 16 * (mt0 + mi) + 4 * q, lane);
#pragma unroll
        for (int ni = 0; ni < S::NTW; ++ni) b[ni] = tr_operand<DV>(vt, klo, khi, 16 * (nt0 + ni) + 4 * q, lane);
#pragma unroll
        for (int mi = 0; mi < S::MTW; ++mi) {
#pragma unroll
            for (int ni = 0; ni < S::NTW; ++ni) st.s[mi][ni] = mfma16x16x32(b[ni], a[mi], st.s[mi][ni]);
            if (mi == zmi) st.z = mfma16x16x32(ones, a[mi], st.z);
        }
        if (vcol) {
#pragma unroll
            for (int ni = 0; ni < S::NTW; ++ni) vc[ni] = mfma16x16x32(b[ni], ones, vc[ni]);
        }
    }
    if (vcol && (lane & 15) == 0) {
#pragma unroll
        for (int ni = 0; ni < S::NTW; ++ni) {
#pragma unroll
            for (int i = 0; i < 4; ++i) vd[16 * (nt0 + ni) + 4 * G + i] = vc[ni][i];
        }
    }
}

// ============================================================== dQ pass
// Per output segment, forward in time from the segment's prefix state.  Wave
// w serves query block qblk (light and heavy blocks paired per SIMD as in the
// forward) and half w % 2 of the key dims.  For elu + 1 the state is carried
// as E = sum elu(k) v^T, zeta = sum elu(k), Vbar = sum v and the token count
// (start: E, zeta and Vbar of the segment's prefix cell; Vbar sits after zeta
// and start_vb may be null for zero); for the identity map E, zeta are S, z.
// The training forward keeps its cells in this same form, so they serve as
// they are.  Writes dq and dd_out (dd of every token, for the dK, dV pass).
// With rev given, a segment p > 0 also sums, over each of R parts j of it
// (sub_chunks chunks each; the library takes the whole segment as one part,
// the granularity the dK, dV pass starts from), dR = phi(Q)^T dY and dr = phi(Q)^T dd
// from the phi(Q), dY and dd it has just staged, into the reverse cell
// (p - 1) R + j at rev + bh rev_stride_bh (cells of Dk Dv + Dk floats, in the
// layout of the forward's segment states); the first segment's are never needed.
template <int DK, int DV, int PHI>
__global__ __launch_bounds__(kThreads8, 1) void bwd_dq8_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ den, const uint16_t *__restrict__ dout, uint16_t *__restrict__ dq,
    float *__restrict__ dd_out, const float *__restrict__ start, size_t start_stride_bh, size_t start_stride_seg,
    const float *__restrict__ start_z, size_t start_z_stride_bh, const float *__restrict__ start_vb, int N, int P,
    int seg_len, float eps, float *__restrict__ rev, size_t rev_stride_bh, int R, int sub_chunks) {
    using TK = Tile<DK>;
    using TV = Tile<DV>;
    constexpr bool KAPPA = PHI == 0; // elu + 1: the constant part is carried apart
    constexpr float kap = KAPPA ? 1.f : 0.f;
    constexpr int FEAT = KAPPA ? kFeatElu : PHI;
    constexpr int KSV = DV / 32;     // k-steps over value dims
    constexpr int NTK = DK / 16 / 2; // key-dim tiles per wave
    // phi(q) (bf16), dY and dd in two buffers, by chunk parity: the reverse
    // sums of a chunk read them after its closing barrier while the next
    // chunk is staged into the other buffer
    __shared__ __attribute__((aligned(16))) uint16_t sQ2[2][kChunk * TK::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * TK::RS]; // features of k (elu for elu + 1)
    __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * TV::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sDY2[2][kChunk * TV::RS];
    __shared__ __attribute__((aligned(16))) float sSq[kChunk];      // sum_i phi(q_i) per row
    __shared__ __attribute__((aligned(16))) float sRed[2 * 2 * kChunk]; // per key-dim half: phi(q).(S dY), phi(q).zeta
    __shared__ __attribute__((aligned(16))) uint16_t sS[DK * DV];
    __shared__ __attribute__((aligned(16))) float sZf[DK];
    __shared__ __attribute__((aligned(16))) float sVb[KAPPA ? DV : 4];     // Vbar before the chunk
    // Vbar in bf16 high and low parts (rows 0 and 1 of an MFMA A operand)
    __shared__ __attribute__((aligned(16))) uint16_t sVbh[KAPPA ? 2 * DV : 8];
    __shared__ __attribute__((aligned(16))) float sVd[KAPPA ? DV : 4]; // the chunk's column sums of V
    __shared__ __attribute__((aligned(16))) float sDD2[2][kChunk];

    const int seg = blockIdx.x % P, bh = blockIdx.x / P;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int l16 = lane & 15, g = lane >> 4, qd = lane & 3;
    const int qblk_w = w < 4 ? (w >> 1) : 5 - (w >> 1), dh = w & 1;
    const bf16x8 ones = bf16_ones8();
    const int t_begin = seg * seg_len;
    const int t_end = min(N, t_begin + seg_len);
    const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
    const size_t row0 = (size_t)bh * N + t_begin;

    State8<DK, DV> st;
    {
        const float *s0 = start ? start + bh * start_stride_bh + seg * start_stride_seg : nullptr;
        const float *z0 = start_z ? start_z + bh * start_z_stride_bh + seg * start_stride_seg : nullptr;
        state8_load<DK, DV>(st, s0, z0, w, lane);
        if (KAPPA && tid < DV) {
            const float *vb0 = start_vb ? start_vb + bh * start_z_stride_bh + seg * start_stride_seg : nullptr;
            const float vb = vb0 ? vb0[tid] : 0.f;
            sVb[tid] = vb;
            const float hi = bf16_round(vb);
            sVbh[tid] = (uint16_t)f32_to_bf16_bits(hi);
            sVbh[DV + tid] = (uint16_t)f32_to_bf16_bits(vb - hi);
        }
    }
    auto state_to_lds = [&] {
        state8_to_lds<DK, DV>(st, sS, w, lane);
        if (State8<DK, DV>::has_z(w) && lane < 16) sZf[State8<DK, DV>::z_dk(w, lane)] = st.z[0];
    };
    state_to_lds();
    // the reverse sums of this segment's state sub-segments (segment 0 has none)
    const bool do_rev = rev != nullptr && seg > 0;
    State8<DK, DV> rt;
    state8_load<DK, DV>(rt, nullptr, nullptr, w, lane);
    auto rev_store = [&](int j) {
        float *dst = rev + bh * rev_stride_bh + ((size_t)(seg - 1) * R + j) * (size_t)(DK * DV + DK);
        state8_store<DK, DV>(rt, dst, w, lane);
        state8_store_z<DK, DV>(rt, dst + DK * DV, w, lane);
    };

    // never negative: a sub-segment may start past the end of a ragged sequence
    auto rows_in = [&](int c) { return max(0, min(kChunk, t_end - t_begin - c * kChunk)); };
    auto issue = [&](BwdBuf<DK, DV, false> &b, int c) {
        const size_t r = row0 + (size_t)c * kChunk;
        b.load(q + r * DK, k + r * DK, v + r * DV, dout + r * DV, den + r, nullptr, rows_in(c), tid);
    };
    // DEPTH chunks of loads in flight: the loads for chunk c + DEPTH are issued
    // while chunk c is worked on (with two, the loop runs two chunks per pass
    // so that each buffer stays in its own registers).  At Dk = Dv = 128 the
    // reverse sums' accumulators leave registers for one.
    constexpr int DEPTH = DK * DV > 64 * 128 ? 1 : 2;
    BwdBuf<DK, DV, false> buf0, buf1;
    // chunk c's tiles into LDS from its buffer, which then takes the loads of
    // chunk c + DEPTH.  The loop stages chunk c + 1 at the end of chunk c's
    // step, after that step's stores: every path into a staging has the same
    // stores after the loads it waits for, so the wait need not cover them.
    auto stage = [&](BwdBuf<DK, DV, false> &buf, const int c) {
        stage_dq<DK, DV, PHI, FEAT>(buf, sQ2[c & 1], sK, sV, sSq, tid);
        stage_dy<DV>(buf.g, buf.den, buf.dd, sDY2[c & 1], nullptr, tid);
        // every read of the buffer before its refill: the loads then land in
        // the buffer's own registers (a load moved above a read would need
        // other registers and a copy back, which waits for it at once).  The
        // refill is not under a branch (past the last chunk its descriptors
        // cover no bytes and the loads read nothing), which would let reads of
        // the buffer sink below it.
        __builtin_amdgcn_sched_barrier(0);
        issue(buf, c + DEPTH);
    };
    issue(buf0, 0);
    if (DEPTH == 2) issue(buf1, 1);
    if (nch > 0) stage(buf0, 0);
    // next: the buffer that holds chunk c + 1
    auto step = [&](BwdBuf<DK, DV, false> &next, const int c) {
        uint16_t *const sQ = sQ2[c & 1];
        uint16_t *const sDY = sDY2[c & 1];
        float *const sDD = sDD2[c & 1];
        const int valid = rows_in(c);
        // the chunk's dq rows and dd, bounded to its valid rows
        const size_t crow = row0 + (size_t)c * kChunk;
        const rsrc_t rdq = chunk_rsrc(dq + crow * DK, valid * DK * 2), rdd = chunk_rsrc(dd_out + crow, valid * 4);
        __syncthreads();
        // tokens before this chunk (the constant part's count)
        const float n_prev = (float)(t_begin + c * kChunk);

        auto chunk_work = [&](auto qblk_c) {
            constexpr int qblk = decltype(qblk_c)::value;
            const int lane = lane_in_loop(tid & 63);
            const int l16 = lane & 15, g = lane >> 4, qd = lane & 3;
            const int tq = 16 * qblk + l16;
            // dY rows of this wave's query block: B operand over value dims
            bf16x8 dya[KSV];
#pragma unroll
            for (int ks = 0; ks < KSV; ++ks)
                dya[ks] = *reinterpret_cast<const bf16x8 *>(sDY + TV::off(tq, 32 * ks + 8 * g));
            // G^T[key][query] = v_key . dY_query for key blocks 0..qblk, zero
            // above the diagonal
            f32x4 gt[4];
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4) {
                gt[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (kb4 <= qblk) {
#pragma unroll
                    for (int ks = 0; ks < KSV; ++ks)
                        gt[kb4] = mfma16x16x32(
                            *reinterpret_cast<const bf16x8 *>(sV + TV::off(16 * kb4 + l16, 32 * ks + 8 * g)), dya[ks],
                            gt[kb4]);
                    // rounded to bf16 here, so that the sum over keys below and
                    // the feat(K)^T G product use the same values (at the first
                    // token the two cancel exactly)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool keep = kb4 < qblk || 4 * g + i <= l16;
                        gt[kb4][i] = keep ? bf16_round(gt[kb4][i]) : 0.f;
                    }
                }
            }
            // Vbar_t . dY_t = Vbar_{c-1} . dY_t + sum_{j <= t} v_j . dY_t, summed in fp32
            float vdy = 0.f;
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4) {
                if (kb4 <= qblk) vdy += (gt[kb4][0] + gt[kb4][1]) + (gt[kb4][2] + gt[kb4][3]);
            }
            if (KAPPA) {
                // Vbar . dY on the matrix cores: rows 0 and 1 of the A operand hold
                // Vbar's bf16 high and low parts (together Vbar to about 2^-17
                // relative; the products accumulate in fp32), so lanes of group 0
                // receive hi . dY and lo . dY (the other rows, and lanes, hold zeros)
                f32x4 vbd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSV; ++ks) {
                    const bf16x8 z8 = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
                    const bf16x8 a = l16 < 2 ? *reinterpret_cast<const bf16x8 *>(sVbh + l16 * DV + 32 * ks + 8 * g) : z8;
                    vbd = mfma16x16x32(a, dya[ks], vbd);
                }
                vdy += vbd[0] + vbd[1];
            }
            vdy = sum_over_groups(vdy);
            // the B operands of the in-chunk products over key steps of 32: G^T
            // (its values are already bf16) and the causal mask itself (bf16
            // ones on and below the diagonal), formed here so that G's fp32
            // accumulators are free before the state product below
            bf16x8 gop[2], mop[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                uint4 u, m;
                u.x = pack_bf16x2(gt[2 * s2][0], gt[2 * s2][1]);
                u.y = pack_bf16x2(gt[2 * s2][2], gt[2 * s2][3]);
                u.z = pack_bf16x2(gt[2 * s2 + 1][0], gt[2 * s2 + 1][1]);
                u.w = pack_bf16x2(gt[2 * s2 + 1][2], gt[2 * s2 + 1][3]);
                auto one = [&](int kb4, int i) -> uint32_t {
                    return kb4 < qblk || (kb4 == qblk && 4 * g + i <= l16) ? 0x3f80u : 0u;
                };
                m.x = one(2 * s2, 0) | one(2 * s2, 1) << 16;
                m.y = one(2 * s2, 2) | one(2 * s2, 3) << 16;
                m.z = one(2 * s2 + 1, 0) | one(2 * s2 + 1, 1) << 16;
                m.w = one(2 * s2 + 1, 2) | one(2 * s2 + 1, 3) << 16;
                gop[s2] = as_bf16x8(u);
                mop[s2] = as_bf16x8(m);
            }

            // A = E_t dY_t and zeta_t over this wave's key dims (tiles permuted as perm_dv)
            f32x4 acc[NTK], zt[NTK];
#pragma unroll
            for (int j = 0; j < NTK; ++j) {
                acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int nt = dh * NTK + j;
                const int dkr = perm_dv(nt, l16);
#pragma unroll
                for (int ks = 0; ks < KSV; ++ks)
                    acc[j] = mfma16x16x32(tiles_row_operand<DV>(sS, dkr, 32 * ks + 8 * g), dya[ks], acc[j]);
                const float4 zf = *reinterpret_cast<const float4 *>(sZf + 32 * (nt >> 1) + 8 * g + 4 * (nt & 1));
                zt[j] = f32x4{zf.x, zf.y, zf.z, zf.w};
            }
            // in-chunk: feat(K)^T Gm^T and feat(K)^T M over key steps of 32
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (2 * s2 <= qblk) {
                    const int klo = 32 * s2 + 4 * g, khi = klo + 16;
#pragma unroll
                    for (int j = 0; j < NTK; ++j) {
                        const int nt = dh * NTK + j;
                        const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
                        const bf16x8 ka = tr_operand<DK>(sK, klo, khi, colq, lane);
                        acc[j] = mfma16x16x32(ka, gop[s2], acc[j]);
                        zt[j] = mfma16x16x32(ka, mop[s2], zt[j]);
                    }
                }
            }
            // phi(q_t) of this lane's key dims: for tile pair p, columns 32 p + 8 g .. + 7
            float fq[NTK][4];
#pragma unroll
            for (int pp = 0; pp < NTK / 2; ++pp) {
                const uint4 r = *reinterpret_cast<const uint4 *>(sQ + TK::off(tq, 32 * (dh * (NTK / 2) + pp) + 8 * g));
                const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    fq[2 * pp][2 * e] = bf_lo(rw[e]);
                    fq[2 * pp][2 * e + 1] = bf_hi(rw[e]);
                    fq[2 * pp + 1][2 * e] = bf_lo(rw[2 + e]);
                    fq[2 * pp + 1][2 * e + 1] = bf_hi(rw[2 + e]);
                }
            }
            // phi(q) . A and phi(q) . zeta over this half of the key dims
            float pa = 0.f, pz = 0.f;
#pragma unroll
            for (int j = 0; j < NTK; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pa = fmaf(fq[j][i], acc[j][i], pa);
                    pz = fmaf(fq[j][i], zt[j][i], pz);
                }
            }
            pa = sum_over_groups(pa);
            pz = sum_over_groups(pz);
            if (g == 0) {
                sRed[(dh * 2 + 0) * kChunk + tq] = pa;
                sRed[(dh * 2 + 1) * kChunk + tq] = pz;
            }
            __syncthreads();
            // dd_t = -phi(q).(S_t dY_t) / (phi(q).z_t + eps) with S = E + 1 Vbar^T,
            // z = zeta + n 1 (kap = 0: S = E, z = zeta)
            const float sq = sSq[tq];
            const float n_t = n_prev + (float)(tq + 1);
            const float num = (sRed[0 * kChunk + tq] + sRed[2 * kChunk + tq]) + kap * sq * vdy;
            const float dnm = (sRed[1 * kChunk + tq] + sRed[3 * kChunk + tq]) + kap * n_t * sq + eps;
            // (the hardware reciprocal, 1 ulp: dphi(q) . phi(q) = num + dd dnm
            // still cancels to the rounding of the terms)
            const float ddq = dnm != 0.f ? -num * __builtin_amdgcn_rcpf(dnm) : 0.f;
            // dphi(q) = A + dd zeta + (Vbar . dY + n dd) 1
            const float cpart = kap * fmaf(n_t, ddq, vdy);
#pragma unroll
            for (int j = 0; j < NTK; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(ddq, zt[j][i], acc[j][i]) + cpart;
            }
            const bool ok = tq < valid;
            const bool dd_lane = dh == 0 && g == 0;
            if (dd_lane) sDD[tq] = ok ? ddq : 0.f;
            buffer_store_f32(ddq, rdd, dd_lane ? tq * 4 : kDropOffset);
            // phi'(q) from the phi(q) values already unpacked for the dot products
#pragma unroll
            for (int j = 0; j < NTK; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[j][i] *= dphi_of<PHI, kScalePhi>(fq[j][i]);
            }
            store_grad_rows<DK, NTK, kScaleNone, PHI>(acc, dh * NTK, nullptr, tq, rdq, g);
        };
        // chunk_work holds one workgroup barrier (the dd exchange), reached by
        // each wave through its own case; as in the delta rule, gfx950's
        // s_barrier counts arriving waves whatever the instruction, and every
        // case executes exactly one.
        switch (qblk_w) {
        case 0: chunk_work(std::integral_constant<int, 0>{}); break;
        case 1: chunk_work(std::integral_constant<int, 1>{}); break;
        case 2: chunk_work(std::integral_constant<int, 2>{}); break;
        default: chunk_work(std::integral_constant<int, 3>{}); break;
        }

        // carry the state across the chunk (elu(0) = 0: rows past the end add
        // nothing; their V rows are zeros)
        if constexpr (KAPPA) {
            state8_update_vcol<DK, DV>(st, sK, sV, w, lane, ones, sVd);
        } else {
            state8_update<DK, DV>(st, sK, sV, w, lane, ones, 0.f);
        }
        __syncthreads();
        if (do_rev) {
            // dR += phi(Q)^T dY, dr += phi(Q)^T dd (rows past the end have dY = 0
            // and dd = 0: nothing to take back out)
            const bf16x8 wop[kChunk / 32] = {dd_operand(sDD, 0, lane >> 4), dd_operand(sDD, 1, lane >> 4)};
            state8_update_w<DK, DV>(rt, sQ, sDY, w, lane, wop, 0.f);
            if ((c + 1) % sub_chunks == 0 || c + 1 == nch) {
                rev_store(c / sub_chunks);
                state8_load<DK, DV>(rt, nullptr, nullptr, w, lane);
            }
        }
        if (c + 1 < nch) {
            state_to_lds();
            if (KAPPA && tid < DV) {
                const float vb = sVb[tid] + sVd[tid];
                sVb[tid] = vb;
                const float hi = bf16_round(vb);
                sVbh[tid] = (uint16_t)f32_to_bf16_bits(hi);
                sVbh[DV + tid] = (uint16_t)f32_to_bf16_bits(vb - hi);
            }
            stage(next, c + 1);
        }
    };
    if constexpr (DEPTH == 2) {
        // two steps per pass, both unconditional (an odd last chunk is peeled)
        // so that each buffer keeps its registers
        int c = 0;
        for (; c + 1 < nch; c += 2) {
            step(buf1, c);
            step(buf0, c + 1);
        }
        if (c < nch) step(buf1, c);
    } else {
        for (int c = 0; c < nch; ++c) step(buf0, c);
    }
    // sub-segments past the end of a ragged sequence: zero cells
    if (do_rev) {
        for (int j = (nch + sub_chunks - 1) / sub_chunks; j < R; ++j) rev_store(j);
    }
}

// ============================================================== dK, dV pass
// Per output segment, backward in time from R, r summed over the later
// segments (zero for the last one).  Wave w serves key block kblk and half
// w % 2 of the key dims (dK) and of the value dims (dV).
template <int DK, int DV, int PHI>
__global__ __launch_bounds__(kThreads8, 1) void bwd_dkv8_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ den, const float *__restrict__ dd, const uint16_t *__restrict__ dout,
    uint16_t *__restrict__ dk, uint16_t *__restrict__ dv, const float *__restrict__ rstart, size_t rstart_stride_bh,
    size_t rstart_stride_seg, int N, int P, int seg_len) {
    using TK = Tile<DK>;
    using TV = Tile<DV>;
    constexpr int KSK = DK / 32, KSV = DV / 32;
    constexpr int NTK = DK / 16 / 2, NTV = DV / 16 / 2;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[kChunk * TK::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * TK::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * TV::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sDY[kChunk * TV::RS];
    __shared__ __attribute__((aligned(16))) float sDD[kChunk];
    __shared__ __attribute__((aligned(16))) uint16_t sR[DK * DV];
    __shared__ __attribute__((aligned(16))) float sRf[DK];

    const int seg = blockIdx.x % P, bh = blockIdx.x / P;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int l16 = lane & 15, g = lane >> 4, qd = lane & 3;
    // key block per wave; blocks 0 (heaviest: every query block follows it)
    // and 3 share a SIMD, as do 1 and 2
    const int kblk_w = w < 4 ? (w >> 1) : 5 - (w >> 1), dh = w & 1;
    const int t_begin = seg * seg_len;
    const int t_end = min(N, t_begin + seg_len);
    const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
    const size_t row0 = (size_t)bh * N + t_begin;

    State8<DK, DV> st; // R^T tiles and r
    {
        const float *r0 = (rstart && seg + 1 < P) ? rstart + bh * rstart_stride_bh + seg * rstart_stride_seg : nullptr;
        state8_load<DK, DV>(st, r0, r0 ? r0 + DK * DV : nullptr, w, lane);
    }
    auto state_to_lds = [&] {
        state8_to_lds<DK, DV>(st, sR, w, lane);
        if (State8<DK, DV>::has_z(w) && lane < 16) sRf[State8<DK, DV>::z_dk(w, lane)] = st.z[0];
    };
    state_to_lds();

    // never negative: a sub-segment may start past the end of a ragged sequence
    auto rows_in = [&](int c) { return max(0, min(kChunk, t_end - t_begin - c * kChunk)); };
    auto issue = [&](BwdBuf<DK, DV> &b, int c) {
        const size_t r = row0 + (size_t)c * kChunk;
        b.load(q + r * DK, k + r * DK, v + r * DV, dout + r * DV, den + r, dd + r, rows_in(c), tid);
    };
    // two chunks in flight, as in the dQ pass
    BwdBuf<DK, DV> buf0, buf1;
    if (nch > 0) issue(buf0, nch - 1);
    if (nch > 1) issue(buf1, nch - 2);
    auto step = [&](BwdBuf<DK, DV> &buf, const int c) {
        const int valid = rows_in(c);
        // the chunk's dk and dv rows, bounded to its valid rows
        const size_t crow = row0 + (size_t)c * kChunk;
        const rsrc_t rdk = chunk_rsrc(dk + crow * DK, valid * DK * 2), rdv = chunk_rsrc(dv + crow * DV, valid * DV * 2);
        stage_qkv<DK, DV, PHI, PHI>(buf, sQ, sK, sV, tid);
        stage_dy<DV>(buf.g, buf.den, buf.dd, sDY, sDD, tid);
        if (c > 1) issue(buf, c - 2);
        __syncthreads();

        auto chunk_work = [&](auto kblk_c) {
            constexpr int kblk = decltype(kblk_c)::value;
            const int lane = lane_in_loop(tid & 63);
            const int l16 = lane & 15, g = lane >> 4, qd = lane & 3;
            const int tk = 16 * kblk + l16;
            auto pack_b = [&](const f32x4(&x)[4], int s2) {
                uint4 u;
                u.x = pack_bf16x2(x[2 * s2][0], x[2 * s2][1]);
                u.y = pack_bf16x2(x[2 * s2][2], x[2 * s2][3]);
                u.z = pack_bf16x2(x[2 * s2 + 1][0], x[2 * s2 + 1][1]);
                u.w = pack_bf16x2(x[2 * s2 + 1][2], x[2 * s2 + 1][3]);
                return as_bf16x8(u);
            };
            // ---- dK: G[query][key] = dY_query . v_key + dd_query (query >= key),
            // then dphi(K)^T = R v^T + r + phi(Q)^T G
            {
                bf16x8 va[KSV];
#pragma unroll
                for (int ks = 0; ks < KSV; ++ks)
                    va[ks] = *reinterpret_cast<const bf16x8 *>(sV + TV::off(tk, 32 * ks + 8 * g));
                f32x4 gq[4];
#pragma unroll
                for (int qb = 0; qb < 4; ++qb) {
                    gq[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (qb >= kblk) {
#pragma unroll
                        for (int ks = 0; ks < KSV; ++ks)
                            gq[qb] = mfma16x16x32(
                                *reinterpret_cast<const bf16x8 *>(sDY + TV::off(16 * qb + l16, 32 * ks + 8 * g)),
                                va[ks], gq[qb]);
                        const float4 dd4 = *reinterpret_cast<const float4 *>(sDD + 16 * qb + 4 * g);
                        const float dda[4] = {dd4.x, dd4.y, dd4.z, dd4.w};
                        // dY . v rounded to bf16 before dd is added: dd was formed
                        // (dQ pass) from these same rounded in-chunk products, and
                        // at the first token dY . v + dd cancels only with them
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bool keep = qb > kblk || 4 * g + i >= l16;
                            gq[qb][i] = keep ? bf16_round(gq[qb][i]) + dda[i] : 0.f;
                        }
                    }
                }
                f32x4 ak[NTK];
#pragma unroll
                for (int j = 0; j < NTK; ++j) {
                    ak[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int nt = dh * NTK + j;
                    const int dkr = perm_dv(nt, l16);
#pragma unroll
                    for (int ks = 0; ks < KSV; ++ks)
                        ak[j] = mfma16x16x32(tiles_row_operand<DV>(sR, dkr, 32 * ks + 8 * g), va[ks], ak[j]);
                    const float4 rf = *reinterpret_cast<const float4 *>(sRf + 32 * (nt >> 1) + 8 * g + 4 * (nt & 1));
                    ak[j][0] += rf.x;
                    ak[j][1] += rf.y;
                    ak[j][2] += rf.z;
                    ak[j][3] += rf.w;
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    if (2 * s2 + 1 >= kblk) {
                        const bf16x8 gop = pack_b(gq, s2);
                        const int klo = 32 * s2 + 4 * g, khi = klo + 16;
#pragma unroll
                        for (int j = 0; j < NTK; ++j) {
                            const int nt = dh * NTK + j;
                            const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
                            ak[j] = mfma16x16x32(tr_operand<DK>(sQ, klo, khi, colq, lane), gop, ak[j]);
                        }
                    }
                }
                store_grad_rows<DK, NTK, kScalePhi, PHI>(ak, dh * NTK, sK, tk, rdk, g);
            }
            // keep the dV phase's loads from being hoisted into the dK phase
            // (they would double the live registers)
            __builtin_amdgcn_sched_barrier(0);
            // ---- dV: P[query][key] = phi(q) . phi(k) (query >= key), then
            // dV^T = R^T phi(k) + dY^T P
            {
                bf16x8 ka[KSK];
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks)
                    ka[ks] = *reinterpret_cast<const bf16x8 *>(sK + TK::off(tk, 32 * ks + 8 * g));
                f32x4 pq[4];
#pragma unroll
                for (int qb = 0; qb < 4; ++qb) {
                    pq[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (qb >= kblk) {
#pragma unroll
                        for (int ks = 0; ks < KSK; ++ks)
                            pq[qb] = mfma16x16x32(
                                *reinterpret_cast<const bf16x8 *>(sQ + TK::off(16 * qb + l16, 32 * ks + 8 * g)),
                                ka[ks], pq[qb]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bool keep = qb > kblk || 4 * g + i >= l16;
                            pq[qb][i] = keep ? pq[qb][i] : 0.f;
                        }
                    }
                }
                f32x4 av[NTV];
#pragma unroll
                for (int j = 0; j < NTV; ++j) {
                    av[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int nt = dh * NTV + j;
                    const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
#pragma unroll
                    for (int ks = 0; ks < KSK; ++ks) {
                        const int klo = 32 * ks + 8 * g;
                        av[j] = mfma16x16x32(tr_operand_in<TileS<DV>>(sR, klo, klo + 4, colq, lane), ka[ks], av[j]);
                    }
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    if (2 * s2 + 1 >= kblk) {
                        const bf16x8 pop = pack_b(pq, s2);
                        const int klo = 32 * s2 + 4 * g, khi = klo + 16;
#pragma unroll
                        for (int j = 0; j < NTV; ++j) {
                            const int nt = dh * NTV + j;
                            const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
                            av[j] = mfma16x16x32(tr_operand<DV>(sDY, klo, khi, colq, lane), pop, av[j]);
                        }
                    }
                }
                store_grad_rows<DV, NTV, kScaleNone, PHI>(av, dh * NTV, nullptr, tk, rdv, g);
            }
        };
        switch (kblk_w) {
        case 0: chunk_work(std::integral_constant<int, 0>{}); break;
        case 1: chunk_work(std::integral_constant<int, 1>{}); break;
        case 2: chunk_work(std::integral_constant<int, 2>{}); break;
        default: chunk_work(std::integral_constant<int, 3>{}); break;
        }

        // carry R, r back across the chunk: R += phi(Q)^T dY, r += phi(Q)^T dd
        const bf16x8 wop[kChunk / 32] = {dd_operand(sDD, 0, lane >> 4), dd_operand(sDD, 1, lane >> 4)};
        state8_update_w<DK, DV>(st, sQ, sDY, w, lane, wop, 0.f);
        __syncthreads();
        if (c > 0) state_to_lds();
    };
    for (int c = nch - 1; c >= 0; c -= 2) {
        step(buf0, c);
        if (c > 0) step(buf1, c - 1);
    }
}

} // namespace linattn
