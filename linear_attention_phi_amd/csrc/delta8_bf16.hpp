// delta8_bf16.hpp -- the delta rule, chunked, eight waves per workgroup, head
// dims Dk, Dv in {64, 128}, bf16 in and out, fp32 state.
//
// Per token ("Linear Attention: what happens when you change the product
// order", section "The summary runs out of room": read with the key before
// writing, write only the difference):
//   kh_t = phi(k_t) / |phi(k_t)|,  S_t = S_{t-1} + beta_t kh_t (v_t - S_{t-1}^T kh_t)^T,
//   o_t  = S_t^T phi(q_t).
// With S_0 the state at a chunk's start and D the chunk's rows
// delta_t = beta_t (v_t - S_{t-1}^T kh_t), expanding S_{t-1} over the chunk
// gives, for the chunk's rows (Kh, Q, V, beta):
//   (I + diag(beta) tril(Kh Kh^T, -1)) D = diag(beta) (V - Kh S_0)
//   O = Q S_0 + tril(Q Kh^T) D      (diagonal included)
//   S_C = S_0 + Kh^T D.
// The unit lower-triangular system is solved in 16-row blocks: the inverses of
// the diagonal blocks by forward substitution in fp32 (one block per wave of
// the light query blocks, as soon as the wave has formed it), the rest as MFMA
// products on bf16 high/low parts; everything else is bf16 MFMA with fp32
// accumulation.  One workgroup carries one (b, h) through its chunks in
// order.  Two kernels: delta8_bf16 (any Dv of 64 and 128; tile layouts and wave
// pairing of fwd8_bf16.hpp, four barriers per chunk: staged, coupled, solved,
// carried) and delta8c_bf16 (Dv = 128: each wave owns 16 value columns of S
// and of every per-column quantity, two barriers per chunk), which the
// library runs at Dv = 128.
#pragma once

#include "bwd8_bf16.hpp"

namespace linattn {

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), eight at a time, as
// MFMA operands (hi carries 8 significant bits, hi + lo about 16).
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
        l[e] = pack_bf16x2(x[2 * e] - bf_lo(h[e]), x[2 * e + 1] - bf_hi(h[e]));
    }
    hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
    lo = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// The same split for four values, as operands of the 16 x 16 x 16 bf16 MFMA.
__device__ __forceinline__ void split_bf16x4(float a, float b, float c, float d, s16x4 &hi, s16x4 &lo) {
    const uint32_t h0 = pack_bf16x2(a, b), h1 = pack_bf16x2(c, d);
    const uint32_t l0 = pack_bf16x2(a - bf_lo(h0), b - bf_hi(h0)), l1 = pack_bf16x2(c - bf_lo(h1), d - bf_hi(h1));
    hi = __builtin_bit_cast(s16x4, make_uint2(h0, h1));
    lo = __builtin_bit_cast(s16x4, make_uint2(l0, l1));
}

// 16 x 16 x 16 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%16][4(l/16)+i],
// B[4(l/16)+i][l%16] and receives C[4(l/16)+i][l%16] (i = 0..3), so a result
// is directly the B operand of a following product over its rows.
__device__ __forceinline__ f32x4 mfma16x16x16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// One value's high and low bf16 parts, as split_bf16x4 forms them.
__device__ __forceinline__ void split_bf16x1(float x, uint16_t &hi, uint16_t &lo) {
    const uint32_t h = f32_to_bf16_bits(x);
    hi = (uint16_t)h;
    lo = (uint16_t)f32_to_bf16_bits(x - __uint_as_float(h << 16));
}

// The solved rows D as bf16 high and low parts, kept in the fp32 right-hand
// side's own rows: the 16 columns 16 m .. 16 m + 15 of a row (64 bytes as
// fp32, owned by one wave in the solve) hold their 16 high parts, then their
// 16 low parts.  Element offsets of the high part; the low part is 16 later.
template <int XS>
struct DSplitTile {
    __device__ static __forceinline__ int off(int r, int c) { return r * (2 * XS) + ((c >> 4) << 5) + (c & 15); }
};

// GATED: the summary is first decayed by a_t (the gated form, Gated DeltaNet).
// With g_t the product of the chunk's gates through t and D(j -> t) the
// product of those after j through t, the chunk's system, outputs and state
// become
//   (I + diag(beta) (tril(Kh Kh^T, -1) o Dec)) D = diag(beta) (V - diag(g) Kh S_0)
//   O = diag(g) Q S_0 + (tril(Q Kh^T) o Dec) D,   S_C = g_C S_0 + Kh^T diag(D(j -> C)) D,
// Dec[t][j] = D(j -> t); exact zeros across a zero gate, as in the gated forward.
template <int DK, int DV, int PHI, bool BETA, bool GATED>
__global__ __launch_bounds__(kThreads8, 1) void delta8_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta, uint16_t *__restrict__ o,
    const float *__restrict__ s_init, float *__restrict__ s_final, int N) {
    using TK = Tile<DK>;
    using TV = Tile<DV>;
    constexpr int KSK = DK / 32;
    constexpr int NTV = DV / 16 / 2; // value tiles per wave
    constexpr int XS = DV + 4;       // fp32 row stride of the right-hand side / solution
    constexpr int AS = kChunk + 4;   // fp32 row stride of the coupling matrix
    __shared__ __attribute__((aligned(16))) uint16_t sQ[kChunk * TK::RS]; // phi(Q)
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * TK::RS]; // unit keys
    __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * TV::RS]; // V, then D (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t sS[DK * DV];         // S_0 in bf16
    __shared__ __attribute__((aligned(16))) float sX[kChunk * XS];        // diag(beta)(V - Kh S_0), then D
    // diag(beta) tril(Kh Kh^T, -1): the diagonal blocks in fp32; below them the
    // negated blocks as bf16 high and low parts, 4 + 4 per 16-byte group
    __shared__ __attribute__((aligned(16))) float sA[kChunk * AS];
    __shared__ __attribute__((aligned(16))) float sB[kChunk]; // beta (0 past the end)
    // inverses of A's diagonal blocks, bf16 high and low parts
    __shared__ __attribute__((aligned(16))) uint16_t sTh[4 * 16 * 16];
    __shared__ __attribute__((aligned(16))) uint16_t sTl[4 * 16 * 16];
    // gated: the chunk's inclusive gate prefix per token (log2 sum, zero count)
    __shared__ __attribute__((aligned(16))) float sGl[GATED ? kChunk : 4];
    __shared__ __attribute__((aligned(16))) int sGz[GATED ? kChunk : 4];

    const size_t bh = blockIdx.x;
    const int tid = threadIdx.x, w = wave_id();
    const int blk_w = w < 4 ? (w >> 1) : 5 - (w >> 1), dh = w & 1;
    const bf16x8 ones = bf16_ones8();
    const int nch = (N + kChunk - 1) / kChunk;
    const size_t row0 = bh * N;

    State8<DK, DV> st;
    state8_load<DK, DV>(st, s_init ? s_init + bh * DK * DV : nullptr, nullptr, w, tid & 63);
    state8_to_lds<DK, DV>(st, sS, w, tid & 63);

    struct Buf {
        Units<DK> q, k;
        Units<DV> v;
        float beta, alpha; // token tid of the chunk (threads below kChunk)
    };
    // rows of chunk c (0 for chunks past the end, whose loads read nothing)
    auto rows_in = [&](int c) { return max(0, min(kChunk, N - c * kChunk)); };
    // every load bounded by a buffer descriptor (0 past the end), none under
    // a branch: beta and alpha of token tid for the threads below kChunk (the
    // others read past the descriptor's end)
    auto issue = [&](Buf &b, int c) {
        const size_t r = row0 + (size_t)c * kChunk;
        const int nv = rows_in(c);
        b.q.load(q + r * DK, nv, tid);
        b.k.load(k + r * DK, nv, tid);
        b.v.load(v + r * DV, nv, tid);
        b.beta = BETA ? buffer_load_f32(chunk_rsrc(beta + r, nv * 4), tid * 4) : (tid < nv ? 1.f : 0.f);
        // (0 past the end: the staging reads no gate of a row past the end)
        b.alpha = GATED ? buffer_load_f32(chunk_rsrc(alpha + r, nv * 4), tid * 4) : 1.f;
    };
    Buf buf;
    // ---- stage chunk c: phi(Q), unit keys (zero past the end), V, beta (and
    // the gate prefix), then refill the buffer with chunk c + 1.  The loop
    // stages chunk c + 1 at the end of chunk c, after that chunk's stores, so
    // that the wait for its loads does not cover the stores.
    auto stage = [&](int c) {
        const int valid = rows_in(c);
        {
            constexpr int CG = Units<DK>::CG;
#pragma unroll
            for (int i = 0; i < Units<DK>::N; ++i) {
                const int row = Units<DK>::row_of(tid, i), col = Units<DK>::col_of(tid, i);
                *reinterpret_cast<uint4 *>(sQ + TK::off(row, col)) = phi_pack8(buf.q.r[i], PHI);
                const uint32_t kw[4] = {buf.k.r[i].x, buf.k.r[i].y, buf.k.r[i].z, buf.k.r[i].w};
                float f[8], nrm = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[2 * e] = phi_fast(bf_lo(kw[e]), PHI);
                    f[2 * e + 1] = phi_fast(bf_hi(kw[e]), PHI);
                    nrm = fmaf(f[2 * e], f[2 * e], fmaf(f[2 * e + 1], f[2 * e + 1], nrm));
                }
                if constexpr (CG == 16) {
                    nrm = row16_sum(nrm);
                } else {
#pragma unroll
                    for (int m = 1; m < CG; m <<= 1) nrm += __shfl_xor(nrm, m, 64);
                }
                // a zero key (or a row past the end) writes nothing; the hardware
                // reciprocal square root (about 1 ulp; the unit key is rounded to
                // bf16 next) in place of a correctly rounded root and division
                const float inv = (row < valid && nrm > 0.f) ? __builtin_amdgcn_rsqf(nrm) : 0.f;
                *reinterpret_cast<uint4 *>(sK + TK::off(row, col)) =
                    make_uint4(pack_bf16x2(f[0] * inv, f[1] * inv), pack_bf16x2(f[2] * inv, f[3] * inv),
                               pack_bf16x2(f[4] * inv, f[5] * inv), pack_bf16x2(f[6] * inv, f[7] * inv));
            }
#pragma unroll
            for (int i = 0; i < Units<DV>::N; ++i)
                *reinterpret_cast<uint4 *>(sV + TV::off(Units<DV>::row_of(tid, i), Units<DV>::col_of(tid, i))) =
                    buf.v.r[i];
            if (tid < kChunk) {
                sB[tid] = buf.beta;
                if (GATED) {
                    ChunkGates cg;
                    cg.build(buf.alpha, tid < valid);
                    sGl[tid] = cg.lsum;
                    sGz[tid] = cg.zeros;
                }
            }
        }
        // every read of the buffer before its refill (a load moved above a
        // read would need other registers and a copy that waits for it)
        __builtin_amdgcn_sched_barrier(0);
        issue(buf, c + 1);
    };
    issue(buf, 0);
    if (nch > 0) stage(0);
    for (int c = 0; c < nch; ++c) {
        const int valid = rows_in(c);
        // the chunk's output rows, bounded to its valid rows
        const rsrc_t ro = chunk_rsrc(o + (row0 + (size_t)c * kChunk) * DV, valid * DV * 2);
        __syncthreads();

        // decay from after token j through token t (j < t), and through t from the chunk's start
        auto dec = [&](int t, int j) { return decay_between(sGl[t], sGz[t], sGl[j], sGz[j]); };
        auto gam = [&](int t) { return decay_between(sGl[t], sGz[t], 0.f, 0); };

        // ---- right-hand side diag(beta)(V - Kh S_0) and the coupling diag(beta) tril(Kh Kh^T, -1)
        {
            const int lane = lane_in_loop(tid & 63);
            const int l16 = lane & 15, g = lane >> 4, qd = lane & 3;
            const int tk = 16 * blk_w + l16; // this wave's keys
            bf16x8 ka[KSK];
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) ka[ks] = *reinterpret_cast<const bf16x8 *>(sK + TK::off(tk, 32 * ks + 8 * g));
            // (Kh S_0)^T tiles: value rows (permuted), key columns
#pragma unroll
            for (int j = 0; j < NTV; ++j) {
                f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
                const int nt = dh * NTV + j;
                const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks) {
                    const int klo = 32 * ks + 8 * g;
                    r = mfma16x16x32(tr_operand_in<TileS<DV>>(sS, klo, klo + 4, colq, lane), ka[ks], r);
                }
                // lane holds key tk, values 32 (nt >> 1) + 8 g + 4 (nt & 1) + i
                const int vc = 32 * (nt >> 1) + 8 * g + 4 * (nt & 1);
                const uint2 vv = *reinterpret_cast<const uint2 *>(sV + TV::off(tk, vc));
                const float b = sB[tk];
                if (GATED) r *= gam(tk);
                *reinterpret_cast<float4 *>(sX + tk * XS + vc) =
                    make_float4(b * (bf_lo(vv.x) - r[0]), b * (bf_hi(vv.x) - r[1]), b * (bf_lo(vv.y) - r[2]),
                                b * (bf_hi(vv.y) - r[3]));
            }
            // coupling blocks: a block (rb, cb) = diag(beta) Kh_rb Kh_cb^T masked
            // below the diagonal; rb = blk_w uses the keys already loaded
            auto gram = [&](int rb, int cb, const bf16x8(&kr)[KSK]) {
                const int tr = 16 * rb + l16;
                f32x4 gr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks)
                    gr = mfma16x16x32(*reinterpret_cast<const bf16x8 *>(sK + TK::off(16 * cb + l16, 32 * ks + 8 * g)),
                                      kr[ks], gr);
                // gr[i] = Kh[16 cb + 4 g + i] . Kh[tr]: the coupling A[tr][j] for
                // j = 16 cb + 4 g + i, strictly below the diagonal
                const float b = sB[tr];
                if (GATED) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = 16 * cb + 4 * g + i;
                        gr[i] *= j < tr ? dec(tr, j) : 0.f;
                    }
                }
                float4 a4;
                a4.x = 16 * cb + 4 * g + 0 < tr ? b * gr[0] : 0.f;
                a4.y = 16 * cb + 4 * g + 1 < tr ? b * gr[1] : 0.f;
                a4.z = 16 * cb + 4 * g + 2 < tr ? b * gr[2] : 0.f;
                a4.w = 16 * cb + 4 * g + 3 < tr ? b * gr[3] : 0.f;
                if (cb == rb) {
                    *reinterpret_cast<float4 *>(sA + tr * AS + 16 * cb + 4 * g) = a4;
                } else {
                    s16x4 hi, lo;
                    split_bf16x4(-a4.x, -a4.y, -a4.z, -a4.w, hi, lo);
                    const uint2 h2 = __builtin_bit_cast(uint2, hi), l2 = __builtin_bit_cast(uint2, lo);
                    *reinterpret_cast<uint4 *>(sA + tr * AS + 16 * cb + 4 * g) = make_uint4(h2.x, h2.y, l2.x, l2.y);
                }
            };
            // waves 0..3 (the light query blocks) take diagonal block w and
            // invert I + A_ww right away, in the wave (lane = column: forward
            // substitution on a unit vector, all four lane groups alike; group
            // g then writes rows 4 g .. 4 g + 3); the six blocks below the
            // diagonal go to waves 4..7
            if (w < 4) {
                const int b = w;
                bf16x8 kd[KSK];
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks)
                    kd[ks] = *reinterpret_cast<const bf16x8 *>(sK + TK::off(16 * b + l16, 32 * ks + 8 * g));
                gram(b, b, kd);
                // this wave wrote the whole block; its LDS accesses stay in order
                const float *ab = sA + 16 * b * AS + 16 * b;
                const int cc = l16;
                float t[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // four partial sums: a short dependency chain per row
                    float x[4] = {r == cc ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j4 = 0; j4 < r; j4 += 4) {
                        const float4 a = *reinterpret_cast<const float4 *>(ab + r * AS + j4);
                        const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (j4 + e < r) x[e] = fmaf(-av[e], t[j4 + e], x[e]);
                    }
                    t[r] = (x[0] + x[1]) + (x[2] + x[3]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * g + i;
                    float tr = t[0];
#pragma unroll
                    for (int rr = 1; rr < 16; ++rr) tr = r == rr ? t[rr] : tr;
                    split_bf16x1(tr, sTh[(16 * b + r) * 16 + cc], sTl[(16 * b + r) * 16 + cc]);
                }
            } else {
                // w = 4, 5: row block 3; w = 6, 7: row block 2 (and w = 7 also
                // block (1, 0), with row block 1's keys)
                if (w == 4) {
                    gram(3, 0, ka);
                    gram(3, 1, ka);
                } else if (w == 5) {
                    gram(3, 2, ka);
                } else {
                    gram(2, w - 6, ka);
                    if (w == 7) {
                        bf16x8 k1[KSK];
#pragma unroll
                        for (int ks = 0; ks < KSK; ++ks)
                            k1[ks] = *reinterpret_cast<const bf16x8 *>(sK + TK::off(16 + l16, 32 * ks + 8 * g));
                        gram(1, 0, k1);
                    }
                }
            }
        }

        // ---- each wave forms the parts of its outputs that do not depend on D
        // (Q S_0 and the masked scores Kh . phi(q); the tiles they read were
        // staged before the last barrier) while the coupling is completed, then
        // solves
        auto chunk_rest = [&](auto blk_c) {
            constexpr int qblk = decltype(blk_c)::value;
            const int lane = lane_in_loop(tid & 63);
            const int l16 = lane & 15, g = lane >> 4, qd = lane & 3;
            const int tq = 16 * qblk + l16;
            // O^T = S_0^T phi(Q)^T (+ the D part below)
            f32x4 acc[NTV];
            // scores^T [key][query] = Kh_key . phi(q)_query, keys at or before the query
            f32x4 sc[4];
            {
                bf16x8 qa[KSK];
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks)
                    qa[ks] = *reinterpret_cast<const bf16x8 *>(sQ + TK::off(tq, 32 * ks + 8 * g));
#pragma unroll
                for (int j = 0; j < NTV; ++j) {
                    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int nt = dh * NTV + j;
                    const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
#pragma unroll
                    for (int ks = 0; ks < KSK; ++ks) {
                        const int klo = 32 * ks + 8 * g;
                        acc[j] = mfma16x16x32(tr_operand_in<TileS<DV>>(sS, klo, klo + 4, colq, lane), qa[ks], acc[j]);
                    }
                    if (GATED) acc[j] *= gam(tq);
                }
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (kb <= qblk) {
#pragma unroll
                        for (int ks = 0; ks < KSK; ++ks)
                            sc[kb] = mfma16x16x32(
                                *reinterpret_cast<const bf16x8 *>(sK + TK::off(16 * kb + l16, 32 * ks + 8 * g)),
                                qa[ks], sc[kb]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if (kb == qblk && 4 * g + i > l16) sc[kb][i] = 0.f;
                            else if (GATED) sc[kb][i] *= dec(tq, 16 * kb + 4 * g + i);
                        }
                    }
                }
            }
            __syncthreads();

            // ---- solve (I + A) D = X: each wave takes 16 value columns through
            // the blocks in order, Y_b = X_b - sum_{k < b} A_bk D_k and
            // D_b = (I + A_bb)^-1 Y_b, as 16 x 16 x 16 MFMAs on bf16 high and low
            // parts (about 16 significant bits), with no workgroup barrier in
            // between.
            if (w < DV / 16) {
                const int col = 16 * w + l16;
                f32x4 dblk[4];
                s16x4 dh4[4], dl4[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    // three independent accumulators (high x high, low x high,
                    // high x low), so the products issue back to back
                    f32x4 y, y1 = f32x4{0.f, 0.f, 0.f, 0.f}, y2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = sX[(16 * b + 4 * g + i) * XS + col];
#pragma unroll
                    for (int kb = 0; kb < b; ++kb) {
                        const uint4 a = *reinterpret_cast<const uint4 *>(sA + (16 * b + l16) * AS + 16 * kb + 4 * g);
                        const s16x4 ah = __builtin_bit_cast(s16x4, make_uint2(a.x, a.y));
                        const s16x4 al = __builtin_bit_cast(s16x4, make_uint2(a.z, a.w));
                        y = mfma16x16x16(ah, dh4[kb], y);
                        y1 = mfma16x16x16(al, dh4[kb], y1);
                        y2 = mfma16x16x16(ah, dl4[kb], y2);
                    }
                    if (b > 0) y += y1 + y2;
                    const uint2 th = *reinterpret_cast<const uint2 *>(sTh + (16 * b + l16) * 16 + 4 * g);
                    const uint2 tl = *reinterpret_cast<const uint2 *>(sTl + (16 * b + l16) * 16 + 4 * g);
                    s16x4 yh, yl;
                    split_bf16x4(y[0], y[1], y[2], y[3], yh, yl);
                    const s16x4 t_h = __builtin_bit_cast(s16x4, th), t_l = __builtin_bit_cast(s16x4, tl);
                    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
                    dblk[b] = mfma16x16x16(t_h, yh, zero) + (mfma16x16x16(t_l, yh, zero) + mfma16x16x16(t_h, yl, zero));
                    split_bf16x4(dblk[b][0], dblk[b][1], dblk[b][2], dblk[b][3], dh4[b], dl4[b]);
                }
                // every read of this wave's right-hand side columns comes before
                // D is written over them
                asm volatile("" ::: "memory");
                // D's high and low parts for the outputs; for the state update
                // each row is decayed to the chunk's end
                uint16_t *sXh = reinterpret_cast<uint16_t *>(sX);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * b + 4 * g + i;
                        const int o = DSplitTile<XS>::off(row, col);
                        sXh[o] = (uint16_t)dh4[b][i];
                        sXh[o + 16] = (uint16_t)dl4[b][i];
                        if (GATED)
                            sV[TV::off(row, col)] = (uint16_t)f32_to_bf16_bits(dblk[b][i] * dec(valid - 1, row));
                        else
                            sV[TV::off(row, col)] = (uint16_t)dh4[b][i];
                    }
                }
            }
            __syncthreads();

            // ---- outputs: O^T += D^T tril(Q Kh^T)^T with both factors split into
            // bf16 high and low parts (three products): the new writes largely
            // cancel the old summary along the keys, and one bf16 rounding of
            // either factor shows in O at the percent level
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (2 * s2 <= qblk) {
                    float x[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = sc[2 * s2][i];
                        x[4 + i] = sc[2 * s2 + 1][i];
                    }
                    bf16x8 bhi, blo;
                    split_bf16x8(x, bhi, blo);
                    const int klo = 32 * s2 + 4 * g, khi = klo + 16;
                    const uint16_t *sXh = reinterpret_cast<const uint16_t *>(sX);
#pragma unroll
                    for (int j = 0; j < NTV; ++j) {
                        const int nt = dh * NTV + j;
                        // this lane's column of D (value perm_dv(nt, l16)), rows klo.. and khi..
                        const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
                        const bf16x8 dhi = tr_operand_in<DSplitTile<XS>>(sXh, klo, khi, colq, lane);
                        const bf16x8 dlo = tr_operand_in<DSplitTile<XS>>(sXh + 16, klo, khi, colq, lane);
                        acc[j] = mfma16x16x32(dhi, bhi, acc[j]);
                        acc[j] = mfma16x16x32(dlo, bhi, acc[j]);
                        acc[j] = mfma16x16x32(dhi, blo, acc[j]);
                    }
                }
            }
            store_grad_rows<DV, NTV, kScaleNone, PHI>(acc, dh * NTV, nullptr, tq, ro, g);
        };
        // chunk_rest holds the chunk's two workgroup barriers, and each wave
        // reaches them through its own case: different s_barrier instructions
        // per wave.  gfx950's s_barrier counts the waves that arrive at any
        // barrier, not a program point, and every case executes exactly two,
        // in the same order relative to the shared LDS traffic, so the waves
        // meet as if at one barrier.  Splitting the phases so that the
        // barriers sit outside the switch measured 2.6% slower (A/B, one
        // process), so the specialization keeps them inside.
        switch (blk_w) {
        case 0: chunk_rest(std::integral_constant<int, 0>{}); break;
        case 1: chunk_rest(std::integral_constant<int, 1>{}); break;
        case 2: chunk_rest(std::integral_constant<int, 2>{}); break;
        default: chunk_rest(std::integral_constant<int, 3>{}); break;
        }
        {
            const int lane = lane_in_loop(tid & 63);
            // S <- g_C S + Kh^T D (rows decayed to the chunk's end; rows past the
            // end have zero keys; z is not used)
            if (GATED) state8_scale<DK, DV>(st, gam(valid - 1));
            state8_update<DK, DV>(st, sK, sV, w, lane, ones, 0.f);
        }
        __syncthreads();
        if (c + 1 < nch) {
            state8_to_lds<DK, DV>(st, sS, w, tid & 63);
            stage(c + 1);
        }
    }
    if (s_final) state8_store<DK, DV>(st, s_final + bh * DK * DV, w, tid & 63);
}

// The same chunked delta rule at Dv = 128 with the value columns owned by the
// waves: wave w keeps S[:, 16 w .. 16 w + 15] in its own registers (lane
// (g, l16) holds four key components of column 16 w + l16 for every key-dim
// tile t, in the order sdk below) and carries its columns through the chunk --
// the right-hand side, the blocked solve, the outputs and the state update --
// with operands taken from its registers.  The waves share only the staged
// tiles, the coupling blocks with their inverses, and the masked scores (as
// bf16 high and low parts), so each chunk has two barriers (staged, shared
// parts formed; the staged tiles are double buffered) and no LDS round trip of
// S, of the right-hand side or of D.
//
// Operand layouts.  An accumulator fragment of two consecutive 16-row tiles
// (lane (g, l16): rows 4 g + i of each, column l16) supplies 8 k values per
// lane group, so it is at once an A operand (rows = its columns) and a B
// operand (columns = its columns) of a 16 x 16 x 32 product, once the other
// operand takes its k values in the same order.  D's rows are keys, taken
// as keys 32 s + 4 g .. + 3, then 32 s + 16 + 4 g .. + 3 (the score tiles
// are stored in that order); the state's rows are key components, kept in an
// order (sdk) that makes them components 32 s + 8 g .. + 7, one 16-byte read
// of a staged row.  S_0 is thus the B operand of Kh S_0 and the A operand of
// S_0^T phi(Q)^T, D the B operand of the state update Kh^T D and the A
// operand of D^T P^T, all straight from the registers that hold them.
template <int DK, int PHI, bool BETA, bool GATED>
__global__ __launch_bounds__(kThreads8, 1) void delta8c_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta, uint16_t *__restrict__ o,
    const float *__restrict__ s_init, float *__restrict__ s_final, int N) {
    constexpr int DV = 128;
    using TK = Tile<DK>;
    using TV = Tile<DV>;
    constexpr int KSK = DK / 32; // 32-component steps over the key dims
    constexpr int NT = DK / 16;  // key-dim tiles of the state
    constexpr int AS = kChunk + 4;
    // the staged tiles in two buffers, by chunk parity: chunk c + 1 is staged
    // while chunk c is still being read
    __shared__ __attribute__((aligned(16))) uint16_t sQb[2][kChunk * TK::RS]; // phi(Q)
    __shared__ __attribute__((aligned(16))) uint16_t sKb[2][kChunk * TK::RS]; // unit keys
    __shared__ __attribute__((aligned(16))) uint16_t sVb[2][kChunk * TV::RS];
    // diag(beta) tril(Kh Kh^T, -1): the diagonal blocks in fp32; below them the
    // negated blocks as bf16 high and low parts, 4 + 4 per 16-byte group
    __shared__ __attribute__((aligned(16))) float sA[kChunk * AS];
    __shared__ __attribute__((aligned(16))) float sBb[2][kChunk]; // beta (0 past the end)
    // inverses of A's diagonal blocks, bf16 high and low parts, each block
    // column-major ([column][row]: a lane writes its column in 16-byte stores)
    __shared__ __attribute__((aligned(16))) uint16_t sTh[4 * 16 * 16];
    __shared__ __attribute__((aligned(16))) uint16_t sTl[4 * 16 * 16];
    // the masked scores P[query][key] as bf16 high (sPh) and low (sPl) parts:
    // per query block qb and key-block pair (2 p, 2 p + 1), p <= qb / 2, the
    // 16 bytes of lane (g, l16) hold keys 16 (2 p) + 4 g .. + 3 then
    // 16 (2 p + 1) + 4 g .. + 3 of query 16 qb + l16 (zeros for the key block
    // past the diagonal): one operand of the outputs' product
    __shared__ __attribute__((aligned(16))) uint4 sPh[6 * 64];
    __shared__ __attribute__((aligned(16))) uint4 sPl[6 * 64];
    __shared__ __attribute__((aligned(16))) float sGlb[2][GATED ? kChunk : 4];
    __shared__ __attribute__((aligned(16))) int sGzb[2][GATED ? kChunk : 4];

    const size_t bh = blockIdx.x;
    const int tid = threadIdx.x, w = wave_id();
    const int nch = (N + kChunk - 1) / kChunk;
    // first key-block pair of query block qb among the six (1, 1, 2, 2 per qb)
    auto pair_base = [](int qb) { return qb == 3 ? 4 : qb; };
    const size_t row0 = bh * N;

    // this wave's columns of the state; the key components of tile t in the
    // order that makes two consecutive tiles' fragments (t = 2 s, 2 s + 1) hold
    // components 32 s + 8 g .. + 7 in lane group g: element i of tile t in
    // group g is component sdk(t, g, i)
    auto sdk = [](int t, int g, int i) { return 32 * (t >> 1) + 8 * g + 4 * (t & 1) + i; };
    f32x4 st[NT];
    {
        const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
        const float *s0 = s_init ? s_init + bh * DK * DV : nullptr;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) st[t][i] = s0 ? s0[sdk(t, g, i) * DV + 16 * w + l16] : 0.f;
        }
    }

    struct Buf {
        Units<DK> q, k;
        Units<DV> v;
        float beta, alpha;
    };
    auto rows_in = [&](int c) { return max(0, min(kChunk, N - c * kChunk)); };
    auto issue = [&](Buf &b, int c) {
        const size_t r = row0 + (size_t)c * kChunk;
        const int nv = rows_in(c);
        b.q.load(q + r * DK, nv, tid);
        b.k.load(k + r * DK, nv, tid);
        b.v.load(v + r * DV, nv, tid);
        b.beta = BETA ? buffer_load_f32(chunk_rsrc(beta + r, nv * 4), tid * 4) : (tid < nv ? 1.f : 0.f);
        b.alpha = GATED ? buffer_load_f32(chunk_rsrc(alpha + r, nv * 4), tid * 4) : 1.f;
    };
    Buf buf;
    // ---- stage chunk c (phi(Q), unit keys, V, beta, the gate prefix), then
    // refill the buffer with chunk c + 1
    auto stage = [&](int c) {
        const int valid = rows_in(c);
        uint16_t *sQ = sQb[c & 1], *sK = sKb[c & 1], *sV = sVb[c & 1];
        float *sB = sBb[c & 1], *sGl = sGlb[c & 1];
        int *sGz = sGzb[c & 1];
        constexpr int CG = Units<DK>::CG;
#pragma unroll
        for (int i = 0; i < Units<DK>::N; ++i) {
            const int row = Units<DK>::row_of(tid, i), col = Units<DK>::col_of(tid, i);
            *reinterpret_cast<uint4 *>(sQ + TK::off(row, col)) = phi_pack8(buf.q.r[i], PHI);
            const uint32_t kw[4] = {buf.k.r[i].x, buf.k.r[i].y, buf.k.r[i].z, buf.k.r[i].w};
            float f[8], nrm = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = phi_fast(bf_lo(kw[e]), PHI);
                f[2 * e + 1] = phi_fast(bf_hi(kw[e]), PHI);
                nrm = fmaf(f[2 * e], f[2 * e], fmaf(f[2 * e + 1], f[2 * e + 1], nrm));
            }
            if constexpr (CG == 16) {
                nrm = row16_sum(nrm);
            } else {
#pragma unroll
                for (int m = 1; m < CG; m <<= 1) nrm += __shfl_xor(nrm, m, 64);
            }
            const float inv = (row < valid && nrm > 0.f) ? __builtin_amdgcn_rsqf(nrm) : 0.f;
            *reinterpret_cast<uint4 *>(sK + TK::off(row, col)) =
                make_uint4(pack_bf16x2(f[0] * inv, f[1] * inv), pack_bf16x2(f[2] * inv, f[3] * inv),
                           pack_bf16x2(f[4] * inv, f[5] * inv), pack_bf16x2(f[6] * inv, f[7] * inv));
        }
#pragma unroll
        for (int i = 0; i < Units<DV>::N; ++i)
            *reinterpret_cast<uint4 *>(sV + TV::off(Units<DV>::row_of(tid, i), Units<DV>::col_of(tid, i))) =
                buf.v.r[i];
        if (tid < kChunk) {
            sB[tid] = buf.beta;
            if (GATED) {
                ChunkGates cg;
                cg.build(buf.alpha, tid < valid);
                sGl[tid] = cg.lsum;
                sGz[tid] = cg.zeros;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(buf, c + 1);
    };
    issue(buf, 0);
    if (nch > 0) stage(0);
    for (int c = 0; c < nch; ++c) {
        const int valid = rows_in(c);
        const rsrc_t ro = chunk_rsrc(o + (row0 + (size_t)c * kChunk) * DV, valid * DV * 2);
        // chunk c staged; chunk c - 1 done with the coupling, inverse and score tiles
        __syncthreads();
        const uint16_t *sQ = sQb[c & 1], *sK = sKb[c & 1], *sV = sVb[c & 1];
        const float *sB = sBb[c & 1], *sGl = sGlb[c & 1];
        const int *sGz = sGzb[c & 1];
        const int lane = lane_in_loop(tid & 63);
        const int l16 = lane & 15, g = lane >> 4, qd = lane & 3;
        auto dec = [&](int t, int j) { return decay_between(sGl[t], sGz[t], sGl[j], sGz[j]); };
        auto gam = [&](int t) { return decay_between(sGl[t], sGz[t], 0.f, 0); };

        // ---- shared parts: the coupling blocks and the inverses of the diagonal
        // ones (wave 0: the four diagonal blocks, then lane group g inverts
        // block g), the six blocks below the diagonal and the ten score tiles
        // (waves 1..7, fewest on wave 4, which shares wave 0's SIMD)
        {
            auto krow = [&](int blk, bf16x8(&kr)[KSK]) {
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks)
                    kr[ks] = *reinterpret_cast<const bf16x8 *>(sK + TK::off(16 * blk + l16, 32 * ks + 8 * g));
            };
            auto gram = [&](int rb, int cb, const bf16x8(&kr)[KSK]) {
                const int tr = 16 * rb + l16;
                f32x4 gr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks)
                    gr = mfma16x16x32(*reinterpret_cast<const bf16x8 *>(sK + TK::off(16 * cb + l16, 32 * ks + 8 * g)),
                                      kr[ks], gr);
                const float b = sB[tr];
                if (GATED) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = 16 * cb + 4 * g + i;
                        gr[i] *= j < tr ? dec(tr, j) : 0.f;
                    }
                }
                float4 a4;
                a4.x = 16 * cb + 4 * g + 0 < tr ? b * gr[0] : 0.f;
                a4.y = 16 * cb + 4 * g + 1 < tr ? b * gr[1] : 0.f;
                a4.z = 16 * cb + 4 * g + 2 < tr ? b * gr[2] : 0.f;
                a4.w = 16 * cb + 4 * g + 3 < tr ? b * gr[3] : 0.f;
                if (cb == rb) {
                    *reinterpret_cast<float4 *>(sA + tr * AS + 16 * cb + 4 * g) = a4;
                } else {
                    s16x4 hi, lo;
                    split_bf16x4(-a4.x, -a4.y, -a4.z, -a4.w, hi, lo);
                    const uint2 h2 = __builtin_bit_cast(uint2, hi), l2 = __builtin_bit_cast(uint2, lo);
                    *reinterpret_cast<uint4 *>(sA + tr * AS + 16 * cb + 4 * g) = make_uint4(h2.x, h2.y, l2.x, l2.y);
                }
            };
            // score tile (qb, kb): P^T[key][query] = Kh . phi(q), masked above
            // the diagonal, decayed between the two tokens when gated
            auto score = [&](int qb, int kb) {
                f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSK; ++ks)
                    sc = mfma16x16x32(*reinterpret_cast<const bf16x8 *>(sK + TK::off(16 * kb + l16, 32 * ks + 8 * g)),
                                      *reinterpret_cast<const bf16x8 *>(sQ + TK::off(16 * qb + l16, 32 * ks + 8 * g)),
                                      sc);
                const int tq = 16 * qb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tk = 16 * kb + 4 * g + i;
                    float x = sc[i];
                    if (GATED) x *= dec(tq, tk);
                    if (kb == qb && tk > tq) x = 0.f;
                    sc[i] = x;
                }
                s16x4 hi, lo;
                split_bf16x4(sc[0], sc[1], sc[2], sc[3], hi, lo);
                const int slot = (pair_base(qb) + (kb >> 1)) * 64 + lane;
                uint2 *ph = reinterpret_cast<uint2 *>(sPh + slot) + (kb & 1);
                uint2 *pl = reinterpret_cast<uint2 *>(sPl + slot) + (kb & 1);
                *ph = __builtin_bit_cast(uint2, hi);
                *pl = __builtin_bit_cast(uint2, lo);
                if (kb == qb && !(kb & 1)) {
                    ph[1] = make_uint2(0u, 0u);
                    pl[1] = make_uint2(0u, 0u);
                }
            };
            if (w == 0) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    bf16x8 kd[KSK];
                    krow(b, kd);
                    gram(b, b, kd);
                }
                // I + A_bb inverted by forward substitution on unit vectors:
                // lane group g takes block g, lane l16 its column l16 (this
                // wave wrote the four blocks; its LDS accesses stay in order)
                const int b = g, cc = l16;
                const float *ab = sA + 16 * b * AS + 16 * b;
                float t[16];
                // four rows at a time: their reads all issued before the
                // substitution steps that use them (so that a step waits for
                // at most one batch of reads, not for each read in turn)
#pragma unroll
                for (int r0 = 0; r0 < 16; r0 += 4) {
                    float4 arow[4][4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
                        for (int j4 = 0; j4 < 4; ++j4)
                            if (4 * j4 < r0 + rr)
                                arow[rr][j4] = *reinterpret_cast<const float4 *>(ab + (r0 + rr) * AS + 4 * j4);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int r = r0 + rr;
                        // four partial sums: a short dependency chain per row
                        float x[4] = {r == cc ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j4 = 0; 4 * j4 < r; ++j4) {
                            const float av[4] = {arow[rr][j4].x, arow[rr][j4].y, arow[rr][j4].z, arow[rr][j4].w};
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (4 * j4 + e < r) x[e] = fmaf(-av[e], t[4 * j4 + e], x[e]);
                        }
                        t[r] = (x[0] + x[1]) + (x[2] + x[3]);
                    }
                }
                uint32_t h[8], lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    h[e] = pack_bf16x2(t[2 * e], t[2 * e + 1]);
                    lo[e] = pack_bf16x2(t[2 * e] - bf_lo(h[e]), t[2 * e + 1] - bf_hi(h[e]));
                }
                uint4 *th = reinterpret_cast<uint4 *>(sTh + (16 * b + cc) * 16);
                uint4 *tl = reinterpret_cast<uint4 *>(sTl + (16 * b + cc) * 16);
                th[0] = make_uint4(h[0], h[1], h[2], h[3]);
                th[1] = make_uint4(h[4], h[5], h[6], h[7]);
                tl[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                tl[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
            } else if (w == 1) {
                bf16x8 kr[KSK];
                krow(1, kr);
                gram(1, 0, kr);
                score(0, 0);
                score(1, 1);
            } else if (w == 2) {
                bf16x8 kr[KSK];
                krow(2, kr);
                gram(2, 0, kr);
                score(1, 0);
                score(2, 2);
            } else if (w == 3) {
                bf16x8 kr[KSK];
                krow(2, kr);
                gram(2, 1, kr);
                score(2, 0);
                score(3, 3);
            } else if (w == 4) {
                bf16x8 kr[KSK];
                krow(3, kr);
                gram(3, 0, kr);
            } else if (w == 5) {
                bf16x8 kr[KSK];
                krow(3, kr);
                gram(3, 1, kr);
                score(2, 1);
                score(3, 0);
            } else if (w == 6) {
                bf16x8 kr[KSK];
                krow(3, kr);
                gram(3, 2, kr);
                score(3, 1);
            } else {
                score(3, 2);
            }
        }

        // ---- this wave's columns before the solve: the right-hand side
        // X = diag(beta)(V - Kh S_0) and the outputs' part O^T = S_0^T phi(Q)^T
        // (S_0 in bf16, as one operand fragment per 32 key components)
        f32x4 x[4], oacc[4];
        {
            bf16x8 sb[KSK];
#pragma unroll
            for (int s = 0; s < KSK; ++s)
                sb[s] = as_bf16x8(make_uint4(pack_bf16x2(st[2 * s][0], st[2 * s][1]),
                                             pack_bf16x2(st[2 * s][2], st[2 * s][3]),
                                             pack_bf16x2(st[2 * s + 1][0], st[2 * s + 1][1]),
                                             pack_bf16x2(st[2 * s + 1][2], st[2 * s + 1][3])));
            // components 32 s + 8 g .. + 7 of a row (the fragment's key components)
            auto row8 = [&](const uint16_t *tile, int row, int s) {
                return *reinterpret_cast<const bf16x8 *>(tile + TK::off(row, 32 * s + 8 * g));
            };
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KSK; ++s) r = mfma16x16x32(row8(sK, 16 * b + l16, s), sb[s], r);
                x[b] = r;
            }
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                // V[16 b + 4 g + i][16 w + l16] for blocks b = 2 b2, 2 b2 + 1
                const bf16x8 vv = tr_operand<DV>(sV, 32 * b2 + 4 * g, 32 * b2 + 16 + 4 * g, 16 * w + 4 * qd, lane);
                const uint4 vu = __builtin_bit_cast(uint4, vv);
                const uint32_t vw[4] = {vu.x, vu.y, vu.z, vu.w};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int b = 2 * b2 + h;
                    const float4 bt = *reinterpret_cast<const float4 *>(sB + 16 * b + 4 * g);
                    const float bv[4] = {bt.x, bt.y, bt.z, bt.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tk = 16 * b + 4 * g + i;
                        const float vi = (i & 1) ? bf_hi(vw[2 * h + (i >> 1)]) : bf_lo(vw[2 * h + (i >> 1)]);
                        float r = x[b][i];
                        if (GATED) r *= gam(tk);
                        x[b][i] = bv[i] * (vi - r);
                    }
                }
            }
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
                f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KSK; ++s) r = mfma16x16x32(sb[s], row8(sQ, 16 * qb + l16, s), r);
                if (GATED) r *= gam(16 * qb + l16);
                oacc[qb] = r;
            }
        }
        // the next chunk into the other buffers (last read by chunk c - 1), before
        // the barrier: the waves that wait there for wave 0's block inverses
        // stage meanwhile
        if (c + 1 < nch) stage(c + 1);
        __syncthreads();

        // ---- solve (I + A) D = X for this wave's columns, block by block:
        // Y_b = X_b - sum_{kb < b} A_b,kb D_kb and D_b = (I + A_bb)^-1 Y_b, as
        // 16 x 16 x 16 products on bf16 high and low parts
        // D's high and low parts, blocks 2 p and 2 p + 1 as the two halves of
        // pair p (the 8 k values of a 16 x 16 x 32 operand)
        f32x4 dblk[4];
        uint4 dH[2], dL[2];
        auto half = [](const uint4 &u, int h) {
            return __builtin_bit_cast(s16x4, h ? make_uint2(u.z, u.w) : make_uint2(u.x, u.y));
        };
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x4 y = x[b], y1 = f32x4{0.f, 0.f, 0.f, 0.f}, y2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < b; ++kb) {
                const uint4 a = *reinterpret_cast<const uint4 *>(sA + (16 * b + l16) * AS + 16 * kb + 4 * g);
                const s16x4 ah = __builtin_bit_cast(s16x4, make_uint2(a.x, a.y));
                const s16x4 al = __builtin_bit_cast(s16x4, make_uint2(a.z, a.w));
                y = mfma16x16x16(ah, half(dH[kb >> 1], kb & 1), y);
                y1 = mfma16x16x16(al, half(dH[kb >> 1], kb & 1), y1);
                y2 = mfma16x16x16(ah, half(dL[kb >> 1], kb & 1), y2);
            }
            if (b > 0) y += y1 + y2;
            // T[16 b + l16][4 g .. + 3] from the column-major block (a
            // transposing read: lane i of a group receives column 4 g + j of row i)
            const int toff = (16 * b + 4 * g + ((lane & 15) >> 2)) * 16 + 4 * qd;
            const uint2 th = lds_tr16(sTh + toff), tl = lds_tr16(sTl + toff);
            s16x4 yh, yl;
            split_bf16x4(y[0], y[1], y[2], y[3], yh, yl);
            const s16x4 t_h = __builtin_bit_cast(s16x4, th), t_l = __builtin_bit_cast(s16x4, tl);
            const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
            dblk[b] = mfma16x16x16(t_h, yh, zero) + (mfma16x16x16(t_l, yh, zero) + mfma16x16x16(t_h, yl, zero));
            s16x4 dh, dl;
            split_bf16x4(dblk[b][0], dblk[b][1], dblk[b][2], dblk[b][3], dh, dl);
            const uint2 hb = __builtin_bit_cast(uint2, dh), lb = __builtin_bit_cast(uint2, dl);
            if (b & 1) {
                dH[b >> 1].z = hb.x, dH[b >> 1].w = hb.y, dL[b >> 1].z = lb.x, dL[b >> 1].w = lb.y;
            } else {
                dH[b >> 1].x = hb.x, dH[b >> 1].y = hb.y, dL[b >> 1].x = lb.x, dL[b >> 1].y = lb.y;
            }
        }

        // ---- outputs: O^T += D^T P^T, both factors in high and low parts
        // (three products: the new writes largely cancel the old summary)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (2 * s2 <= qb) {
                    const int slot = (pair_base(qb) + s2) * 64 + lane;
                    const bf16x8 phi8 = as_bf16x8(sPh[slot]), plo8 = as_bf16x8(sPl[slot]);
                    const bf16x8 dhi = as_bf16x8(dH[s2]), dlo = as_bf16x8(dL[s2]);
                    oacc[qb] = mfma16x16x32(dhi, phi8, oacc[qb]);
                    oacc[qb] = mfma16x16x32(dlo, phi8, oacc[qb]);
                    oacc[qb] = mfma16x16x32(dhi, plo8, oacc[qb]);
                }
            }
            // lane (g, l16): O[16 qb + l16][16 w + 4 g .. + 3]
            const uint2 u = make_uint2(pack_bf16x2(oacc[qb][0], oacc[qb][1]), pack_bf16x2(oacc[qb][2], oacc[qb][3]));
            buffer_store8(u, ro, ((16 * qb + l16) * DV + 16 * w + 4 * g) * 2);
        }

        // ---- S <- g_C S + Kh^T D for this wave's columns (rows of D decayed to
        // the chunk's end when gated; rows past the end have zero keys)
        {
            uint4 du[2] = {dH[0], dH[1]};
            if (GATED) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int tk0 = 16 * b + 4 * g;
                    const float e0 = dblk[b][0] * dec(valid - 1, tk0), e1 = dblk[b][1] * dec(valid - 1, tk0 + 1);
                    const float e2 = dblk[b][2] * dec(valid - 1, tk0 + 2), e3 = dblk[b][3] * dec(valid - 1, tk0 + 3);
                    if (b & 1)
                        du[b >> 1].z = pack_bf16x2(e0, e1), du[b >> 1].w = pack_bf16x2(e2, e3);
                    else
                        du[b >> 1].x = pack_bf16x2(e0, e1), du[b >> 1].y = pack_bf16x2(e2, e3);
                }
            }
            if (GATED) {
                const float gc = gam(valid - 1);
#pragma unroll
                for (int t = 0; t < NT; ++t) st[t] *= gc;
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const bf16x8 db = as_bf16x8(du[s2]);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    st[t] = mfma16x16x32(tr_operand<DK>(sK, 32 * s2 + 4 * g, 32 * s2 + 16 + 4 * g,
                                                        32 * (t >> 1) + 8 * qd + 4 * (t & 1), lane),
                                         db, st[t]);
            }
        }
    }
    if (s_final) {
        const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
        float *sf = s_final + bh * DK * DV;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sf[sdk(t, g, i) * DV + 16 * w + l16] = st[t][i];
        }
    }
}

} // namespace linattn
