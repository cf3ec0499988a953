// fwd8_bf16.hpp -- chunked causal linear attention, eight-wave version for
// head dims Dk, Dv in {64, 128} (bf16 inputs, bf16 MFMA, fp32 state).
//
// Same algebra as fwd_bf16.hpp (per 64-token chunk: scores tril(phi(Q) phi(K)^T),
// in-chunk output, read of the carried summary, state update), arranged for
// gfx950:
//  * 8 waves per workgroup (two per SIMD) so matrix, vector and LDS work of
//    one wave overlaps the other's;
//  * all chunk data sits in LDS row-major, [token][d], written with 16-byte
//    stores; the token-contiguous operands of the contractions over tokens
//    (phi(K)^T, V^T and V) are read with the gfx950 transposing LDS load
//    ds_read_b64_tr_b16 instead of being written transposed;
//  * rows are padded by 32 elements and their 16-byte chunks XOR-swizzled by
//    row, which keeps the row reads, the transposing reads and the S^T copy at
//    the minimum number of LDS cycles;
//  * phi is evaluated once per element, V is staged without conversion.
#pragma once

#include "common.hpp"
#include "fwd_bf16.hpp"

namespace linattn {

typedef short v4i16 __attribute__((ext_vector_type(4)));
constexpr int kThreads8 = 512;

// Row-major bf16 tile in LDS with D + 32 elements per row and the 16-byte
// chunk index XOR-ed with 2 * ((row >> 3) & 3).  Element offsets; columns
// accessed in groups of 4 or 8 stay contiguous.
template <int D>
struct Tile {
    static constexpr int RS = D + 32;
    __device__ static __forceinline__ int off(int r, int c) {
        return r * RS + ((((c >> 3) ^ (((r >> 3) & 3) << 1)) << 3) | (c & 7));
    }
};

// The bf16 copy of the state S in LDS: [dk][dv], Dv elements per row, no
// padding, its 8-byte groups of 4 elements XOR-swizzled by a GF(2)-linear map
// of row bits 0..3 (images 1, C1, 2, C3).  It is written 8 bytes per lane from
// the S^T accumulators (16 consecutive rows per group of 16 lanes) and read
// with the transposing load as the S^T operand of the summary read, whose
// value columns are permuted as in perm_dv.  With 32 LDS banks serving each
// 16-lane group of a 64-bit write and 64 banks each half-wave of a 64-bit
// read, the map puts both patterns on distinct banks (for Dv = 128 and 64).
template <int DV>
struct TileS {
    static_assert(DV == 64 || DV == 128, "TileS covers Dv = 64 and 128");
    static constexpr int G = DV / 4;
    static constexpr int C1 = DV == 128 ? 8 : 5, C3 = DV == 128 ? 20 : 8;
    __device__ static __forceinline__ int sw(int r) {
        return (r & 1) ^ ((r & 2) ? C1 : 0) ^ ((r & 4) ? 2 : 0) ^ ((r & 8) ? C3 : 0);
    }
    // element offset of (r, c); c % 4 is kept, so 4-element groups stay contiguous
    __device__ static __forceinline__ int off(int r, int c) {
        return r * DV + ((((c >> 2) ^ sw(r)) & (G - 1)) << 2) + (c & 3);
    }
};

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 4-element segments addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ uint2 lds_tr16(const uint16_t *p) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
    return __builtin_bit_cast(uint2, v);
}

// MFMA operand with k along the rows of a row-major tile M[k][col]:
// lane (G = lane >> 4, i = lane & 15) receives M[klo + j][col_i] (j = 0..3)
// then M[khi + j][col_i] (j = 0..3), where col_i = colq(i / 4) + i % 4.  Each
// lane passes klo / khi of its own group and colq of its own quad (lane & 3).
template <typename L>
__device__ __forceinline__ bf16x8 tr_operand_in(const uint16_t *tile, int klo, int khi, int colq, int lane) {
    const int src = lane & 15;
    const uint2 a = lds_tr16(tile + L::off(klo + (src >> 2), colq));
    const uint2 b = lds_tr16(tile + L::off(khi + (src >> 2), colq));
    return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *tile, int klo, int khi, int colq, int lane) {
    return tr_operand_in<Tile<D>>(tile, klo, khi, colq, lane);
}

// phi of 8 packed bf16 values.  Rows past the end of the sequence are not
// masked here: their V rows are zero and causality hides their keys from every
// valid query; only z takes them back out (state8_update).
__device__ __forceinline__ uint4 phi_pack8(uint4 raw, int phi_mode) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint4 o;
    uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
    for (int e = 0; e < 4; ++e) ow[e] = pack_bf16x2(phi_fast(bf_lo(w[e]), phi_mode), phi_fast(bf_hi(w[e]), phi_mode));
    return o;
}

// The same, written both plain and scaled (one phi, two packs).
__device__ __forceinline__ void phi_pack8x2(uint4 raw, int phi_mode, float scale, uint4 &plain, uint4 &scaled) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t *op = reinterpret_cast<uint32_t *>(&plain);
    uint32_t *os = reinterpret_cast<uint32_t *>(&scaled);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float lo = phi_fast(bf_lo(w[e]), phi_mode), hi = phi_fast(bf_hi(w[e]), phi_mode);
        op[e] = pack_bf16x2(lo, hi);
        os[e] = pack_bf16x2(lo * scale, hi * scale);
    }
}

// Per-thread share of a 64 x D chunk: units of 8 columns of one row, unit
// u = tid + 512 r -> row u / (D / 8), column group u % (D / 8).  A chunk is
// contiguous (rows of D elements), so unit u sits at byte 16 u of it.
template <int D>
struct Units {
    static constexpr int CG = D / 8;
    static constexpr int N = kChunk * CG / kThreads8;
    uint4 r[N];
    // Buffer loads bounded to the chunk's valid rows: rows past the end read
    // as zero with no per-row compare, select or branch, and the descriptor
    // (base, size) lives in scalar registers.  The state pass streams its
    // reads past the caches (load_stream); the output pass reads with the
    // default policy (load), which measured faster there.
    template <bool STREAM>
    __device__ __forceinline__ void load_policy(const uint16_t *__restrict__ base, int rows_valid, int tid) {
        const rsrc_t rs = chunk_rsrc(base, rows_valid * D * 2);
#pragma unroll
        for (int i = 0; i < N; ++i) r[i] = buffer_load16<STREAM>(rs, (tid + kThreads8 * i) * 16);
    }
    __device__ __forceinline__ void load(const uint16_t *base, int rows_valid, int tid) {
        load_policy<false>(base, rows_valid, tid);
    }
    __device__ __forceinline__ void load_stream(const uint16_t *base, int rows_valid, int tid) {
        load_policy<true>(base, rows_valid, tid);
    }
    __device__ static __forceinline__ int row_of(int tid, int i) { return (tid + kThreads8 * i) / CG; }
    __device__ static __forceinline__ int col_of(int tid, int i) { return ((tid + kThreads8 * i) % CG) * 8; }
};

// State tiles of one wave: 2 x 4 wave grid over (Dk, Dv), held transposed:
// the accumulator of tile (mi, ni) is S^T over value rows 16 nt + 4 g + i and
// key columns 16 mt + l16, so lane (g, l16) holds S[dk][dv .. dv + 3] with
// dk = 16 mt + l16, dv = 16 nt + 4 g.  z is one more accumulator: wave w with
// w % 4 below MTW accumulates 1^T phi(K) for its key-dimension tile
// mt0 + w % 4 (reusing the phi(K) operand its state update already holds), so
// every element of lane l16 holds z[16 (mt0 + w % 4) + l16].
template <int DK, int DV>
struct State8 {
    static constexpr int MT = DK / 16, NT = DV / 16;
    static constexpr int MTW = MT / 2, NTW = NT / 4;
    f32x4 s[MTW][NTW];
    f32x4 z;
    __device__ static __forceinline__ int zmi(int w) { return w & 3; }
    __device__ static __forceinline__ bool has_z(int w) { return (w & 3) < MTW; }
    // the key dimension whose z this lane holds
    __device__ static __forceinline__ int z_dk(int w, int lane) { return 16 * ((w >> 2) * MTW + (w & 3)) + (lane & 15); }
};

// s: [Dk][Dv] (or null for zeros); z: [Dk] (or null for zeros).
template <int DK, int DV>
__device__ __forceinline__ void state8_load(State8<DK, DV> &st, const float *s, const float *z, int w, int lane) {
    using S = State8<DK, DV>;
    const int l16 = lane & 15, g = lane >> 4, mt0 = (w >> 2) * S::MTW, nt0 = (w & 3) * S::NTW;
#pragma unroll
    for (int mi = 0; mi < S::MTW; ++mi) {
#pragma unroll
        for (int ni = 0; ni < S::NTW; ++ni) {
            const float *p = s ? s + (size_t)(16 * (mt0 + mi) + l16) * DV + 16 * (nt0 + ni) + 4 * g : nullptr;
#pragma unroll
            for (int i = 0; i < 4; ++i) st.s[mi][ni][i] = p ? p[i] : 0.f;
        }
    }
    const float zv = z && S::has_z(w) ? z[S::z_dk(w, lane)] : 0.f;
    st.z = f32x4{zv, zv, zv, zv};
}

template <int DK, int DV>
__device__ __forceinline__ void state8_store(const State8<DK, DV> &st, float *s, int w, int lane) {
    using S = State8<DK, DV>;
    const int l16 = lane & 15, g = lane >> 4, mt0 = (w >> 2) * S::MTW, nt0 = (w & 3) * S::NTW;
#pragma unroll
    for (int mi = 0; mi < S::MTW; ++mi) {
#pragma unroll
        for (int ni = 0; ni < S::NTW; ++ni) {
            float *p = s + (size_t)(16 * (mt0 + mi) + l16) * DV + 16 * (nt0 + ni) + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = st.s[mi][ni][i];
        }
    }
}

// z of this wave's tile to z[Dk] (lanes 0..15 of the waves holding z).
template <int DK, int DV>
__device__ __forceinline__ void state8_store_z(const State8<DK, DV> &st, float *z, int w, int lane) {
    using S = State8<DK, DV>;
    if (S::has_z(w) && lane < 16) z[S::z_dk(w, lane)] = st.z[0];
}

// z in bf16 into a plain row of Dk elements (lanes 0..15 of the z waves).
template <int DK, int DV>
__device__ __forceinline__ void state8_z_to_lds(const State8<DK, DV> &st, uint16_t *zrow, int w, int lane) {
    using S = State8<DK, DV>;
    if (S::has_z(w) && lane < 16) zrow[S::z_dk(w, lane)] = (uint16_t)f32_to_bf16_bits(st.z[0]);
}

template <int DK, int DV>
__device__ __forceinline__ void state8_scale(State8<DK, DV> &st, float d) {
    using S = State8<DK, DV>;
#pragma unroll
    for (int mi = 0; mi < S::MTW; ++mi) {
#pragma unroll
        for (int ni = 0; ni < S::NTW; ++ni) st.s[mi][ni] *= d;
    }
    st.z *= d;
}

// S += phi(K)^T V and z += phi(K)^T w over one chunk for this wave's tiles
// (as S^T += V^T phi(K): the V operand supplies the rows, phi(K) the columns).
// kt: phi(K) rows (decayed to the chunk end when gated), vt: V rows; wop[ks]:
// the per-token weights of z for the 32 tokens of step ks in this lane's
// operand order (all ones for z itself).  Rows past the end of the sequence
// hold phi(0) in kt and zeros in vt: they add nothing to S, and pad (their
// weighted count times phi(0)) is taken back out of z.
template <int DK, int DV>
__device__ __forceinline__ void state8_update_w(State8<DK, DV> &st, const uint16_t *kt, const uint16_t *vt, int w,
                                                int lane, const bf16x8 (&wop)[kChunk / 32], float pad) {
    using S = State8<DK, DV>;
    const int G = lane >> 4, q = lane & 3, mt0 = (w >> 2) * S::MTW, nt0 = (w & 3) * S::NTW;
    const int zmi = S::zmi(w);
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
            if (mi == zmi) st.z = mfma16x16x32(wop[ks], a[mi], st.z);
        }
    }
    st.z -= pad;
}

template <int DK, int DV>
__device__ __forceinline__ void state8_update(State8<DK, DV> &st, const uint16_t *kt, const uint16_t *vt, int w,
                                              int lane, bf16x8 ones, float pad) {
    const bf16x8 wop[kChunk / 32] = {ones, ones};
    state8_update_w<DK, DV>(st, kt, vt, w, lane, wop, pad);
}

// bf16 S [dk][dv] into LDS (TileS layout): each lane writes the four values
// dv .. dv + 3 of row dk of each of its tiles.
template <int DK, int DV>
__device__ __forceinline__ void state8_to_lds(const State8<DK, DV> &st, uint16_t *sS, int w, int lane) {
    using S = State8<DK, DV>;
    const int l16 = lane & 15, g = lane >> 4, mt0 = (w >> 2) * S::MTW, nt0 = (w & 3) * S::NTW;
#pragma unroll
    for (int mi = 0; mi < S::MTW; ++mi) {
#pragma unroll
        for (int ni = 0; ni < S::NTW; ++ni) {
            uint2 u;
            u.x = pack_bf16x2(st.s[mi][ni][0], st.s[mi][ni][1]);
            u.y = pack_bf16x2(st.s[mi][ni][2], st.s[mi][ni][3]);
            *reinterpret_cast<uint2 *>(sS + TileS<DV>::off(16 * (mt0 + mi) + l16, 16 * (nt0 + ni) + 4 * g)) = u;
        }
    }
}

// Column sums of staged Units<D> rows: vsum[e] += element e of the unit, in fp32.
__device__ __forceinline__ void add_bf16x8(float (&vsum)[8], uint4 u) {
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        vsum[2 * e] += bf_lo(wv[e]);
        vsum[2 * e + 1] += bf_hi(wv[e]);
    }
}

// Per-thread column sums of Units<D> (columns 8 (tid % (D / 8)) + e) summed
// over the wave's lanes with the same columns, then written as this wave's
// row of red[8][D] (lanes 0 .. D / 8 - 1).
template <int D>
__device__ __forceinline__ void colsum_to_lds(float (&vsum)[8], float *red, int w, int lane) {
    constexpr int CG = D / 8;
    if constexpr (CG == 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vsum[e] = sum_over_groups(vsum[e]);
    } else {
#pragma unroll
        for (int m = CG; m < 64; m <<= 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) vsum[e] += __shfl_xor(vsum[e], m, 64);
        }
    }
    if (lane < CG) {
        float4 *r = reinterpret_cast<float4 *>(red + w * D + 8 * lane);
        r[0] = make_float4(vsum[0], vsum[1], vsum[2], vsum[3]);
        r[1] = make_float4(vsum[4], vsum[5], vsum[6], vsum[7]);
    }
}

// Column col of the eight waves' rows of red[8][D], summed in wave order.
template <int D>
__device__ __forceinline__ float colsum_from_lds(const float *red, int col) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) x += red[w * D + col];
    return x;
}

// ====================================================================== kernels
// Carry a state over tokens [t_begin, t_end) of head bh: st holds the state
// before t_begin on entry and the state after t_end - 1 on return (gated: the
// decay of each chunk applies to what st held).  The range's gate log2-sum
// and zero count are added to seg_lsum, seg_zeros; with VBAR, the column sums
// of this thread's V units are added to vsum (the unit layout repeats every
// 512 units, so a thread's columns are the same in every chunk).  Two
// workgroups share a compute unit, so one chunk of loads in flight per
// workgroup (refilled as soon as it is staged) keeps both fed.
template <int DK, int DV, bool GATED, int PHI, bool VBAR>
__device__ __forceinline__ void range_state8(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                             const float *__restrict__ alpha, size_t bh, int N, int t_begin,
                                             int t_end, State8<DK, DV> &st, uint16_t *sK, uint16_t *sV,
                                             float (&vsum)[8], float &seg_lsum, int &seg_zeros) {
    constexpr int phi_mode = PHI;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
    const uint16_t *kb = k + (bh * N + t_begin) * DK;
    const uint16_t *vb = v + (bh * N + t_begin) * DV;
    const float *ab = GATED ? alpha + bh * N + t_begin : nullptr;
    const bf16x8 ones = bf16_ones8();

    struct Buf {
        Units<DK> k;
        Units<DV> v;
        float a;
    };
    auto rows_in = [&](int c) { return min(kChunk, t_end - t_begin - c * kChunk); };
    auto issue = [&](Buf &b, int c) {
        const int nv = rows_in(c);
        b.k.load_stream(kb + (size_t)c * kChunk * DK, nv, tid);
        b.v.load_stream(vb + (size_t)c * kChunk * DV, nv, tid);
        if (GATED) b.a = lane < nv ? ab[c * kChunk + lane] : 1.f;
    };
    auto step = [&](Buf &b, int c) {
        const int valid = rows_in(c);
        float dC = 1.f, ke = 0.f;
        ChunkGates cg;
        if (GATED) {
            cg.build(b.a, lane < valid);
            seg_lsum += cg.lsum_at(valid - 1);
            seg_zeros += cg.zeros_at(valid - 1);
            ke = cg.kappa_at(valid - 1);
            dC = decay_k(ke, 0.f);
        }
#pragma unroll
        for (int i = 0; i < Units<DK>::N; ++i) {
            const int row = Units<DK>::row_of(tid, i);
            const float sc = GATED ? decay_k(ke, cg.kappa_at(row)) : 1.f;
            uint4 plain, scaled;
            phi_pack8x2(b.k.r[i], phi_mode, sc, plain, scaled);
            *reinterpret_cast<uint4 *>(sK + Tile<DK>::off(row, Units<DK>::col_of(tid, i))) = GATED ? scaled : plain;
        }
#pragma unroll
        for (int i = 0; i < Units<DV>::N; ++i) {
            *reinterpret_cast<uint4 *>(sV + Tile<DV>::off(Units<DV>::row_of(tid, i), Units<DV>::col_of(tid, i))) =
                b.v.r[i];
            if (VBAR) add_bf16x8(vsum, b.v.r[i]);
        }
        if (c + 1 < nch) issue(b, c + 1);
        __syncthreads();
        if (GATED) state8_scale<DK, DV>(st, dC);
        state8_update<DK, DV>(st, sK, sV, w, lane, ones, phi_mode ? 0.f : (float)(kChunk - valid));
        __syncthreads();
    };
    if (nch > 0) {
        Buf b0;
        issue(b0, 0);
        for (int c = 0; c < nch; ++c) step(b0, c);
    }
}

// Segment-state pass (see seg_state_bf16): dS = phi(K)^T V and dz over one
// state sub-segment, plus the segment's gate product.
// PHI: the feature map (0: elu + 1, 1: identity, kFeatElu: elu), fixed at
// compile time so that phi costs no per-element select.  VBAR: the cell also
// holds the column sums of V (Dv more floats after z), the constant part of
// the state when the features are written 1 + elu.
template <int DK, int DV, bool GATED, int PHI, bool VBAR = false>
__global__ __launch_bounds__(kThreads8, 4) void seg_state8_bf16(const uint16_t *__restrict__ k,
                                                                const uint16_t *__restrict__ v,
                                                                const float *__restrict__ alpha,
                                                                float *__restrict__ ws, float *__restrict__ gam, int N,
                                                                int P, int P_run, int seg_len) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * Tile<DK>::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * Tile<DV>::RS];

    const int seg = blockIdx.x % P_run, bh = blockIdx.x / P_run;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int t_begin = seg * seg_len;
    const int t_end = min(N, t_begin + seg_len);

    State8<DK, DV> st;
    state8_load<DK, DV>(st, nullptr, nullptr, w, lane);
    float seg_lsum = 0.f;
    int seg_zeros = 0;
    float vsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    range_state8<DK, DV, GATED, PHI, VBAR>(k, v, alpha, bh, N, t_begin, t_end, st, sK, sV, vsum, seg_lsum,
                                           seg_zeros);
    constexpr size_t E = (size_t)DK * DV + DK + (VBAR ? DV : 0);
    float *dst = ws + ((size_t)bh * P + seg) * E;
    state8_store<DK, DV>(st, dst, w, lane);
    state8_store_z<DK, DV>(st, dst + DK * DV, w, lane);
    if (VBAR) {
        // sK is free after the last chunk's closing barrier
        float *red = reinterpret_cast<float *>(sK);
        colsum_to_lds<DV>(vsum, red, w, lane);
        __syncthreads();
        if (tid < DV) dst[DK * DV + DK + tid] = colsum_from_lds<DV>(red, tid);
    }
    if (GATED && tid == 0) gam[(size_t)bh * P + seg] = seg_zeros > 0 ? 0.f : __builtin_amdgcn_exp2f(seg_lsum);
}

// Snapshot positions of one call (the same for every (b, h)), passed by value
// in the kernel arguments.
constexpr int kMaxSnapshots = 256;
struct SnapList {
    int n;
    int pos[kMaxSnapshots];
};

// State snapshots: (S, z) after token p for each listed p, written to
// s_snap [BH][n][Dk][Dv] and z_snap [BH][n][Dk].  Each workgroup starts from
// the last prefix cell at or before token p + 1 (cells of cell_len tokens,
// the last one usable is max_cell, which may be the end of the sequence;
// null cells: the initial state or zero at token 0) and carries the state
// over the tokens from there through p, the forward's own algebra (gated: the
// decays of those tokens apply to the cell's state).  Without gates, when the
// next cell is nearer, it takes that cell's state less the sums of the tokens
// after p instead (the sums are additive; negating the cell, adding the
// tokens and negating again is exact up to the additions' rounding).  A
// snapshot just before a cell edge is a copy of the cell.
template <int DK, int DV, bool GATED, int PHI>
__global__ __launch_bounds__(kThreads8, 4) void snap_state8_bf16(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const float *__restrict__ alpha,
    const float *__restrict__ cells, size_t cell_stride_bh, int cell_len, int max_cell,
    const float *__restrict__ s_init, const float *__restrict__ z_init, float *__restrict__ s_snap,
    float *__restrict__ z_snap, int N, SnapList snaps) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * Tile<DK>::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * Tile<DV>::RS];

    const int i = blockIdx.x % snaps.n, bh = blockIdx.x / snaps.n;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int p = snaps.pos[i];
    int cell = cells ? min((p + 1) / cell_len, max_cell) : 0;
    int t_begin = cell * cell_len, t_end = p + 1;
    // the next cell and its token, when it is nearer (ungated only)
    bool back = false;
    if (!GATED && cells && cell + 1 <= max_cell) {
        const int hi_tok = min((cell + 1) * cell_len, N);
        if (hi_tok - (p + 1) < (p + 1) - t_begin) {
            back = true;
            cell += 1;
            t_begin = p + 1;
            t_end = hi_tok;
        }
    }

    State8<DK, DV> st;
    if (cells) {
        const float *c0 = cells + bh * cell_stride_bh + (size_t)cell * (DK * DV + DK);
        state8_load<DK, DV>(st, c0, c0 + DK * DV, w, lane);
    } else {
        state8_load<DK, DV>(st, s_init ? s_init + (size_t)bh * DK * DV : nullptr,
                            z_init ? z_init + (size_t)bh * DK : nullptr, w, lane);
    }
    if (back) state8_scale<DK, DV>(st, -1.f);
    float seg_lsum = 0.f;
    int seg_zeros = 0;
    float vsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    range_state8<DK, DV, GATED, PHI, false>(k, v, alpha, bh, N, t_begin, t_end, st, sK, sV, vsum, seg_lsum,
                                            seg_zeros);
    if (back) state8_scale<DK, DV>(st, -1.f);
    const size_t o = (size_t)bh * snaps.n + i;
    state8_store<DK, DV>(st, s_snap + o * DK * DV, w, lane);
    state8_store_z<DK, DV>(st, z_snap + o * DK, w, lane);
}

// Causal output pass (see fwd_out_bf16): wave w serves query block w / 2 and
// half w % 2 of the value columns; the state tiles are split 2 x 4.  TRAIN:
// also keep, for the backward, each token's denominator phi(q).z + eps
// (den_out).  start_vb non-null (training, elu + 1): the start cells hold the
// backward's form, E = sum elu(k) v^T and zeta = sum elu(k) (plus any initial
// state), with the column sums of V at start_vb; the state is then
// S = E + 1 Vbar^T, z = zeta + n 1, n the tokens before the segment.
template <int DK, int DV, bool GATED, int PHI, bool TRAIN = false>
__global__ __launch_bounds__(kThreads8, 1) void fwd_out8_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, uint16_t *__restrict__ o, const float *__restrict__ start, size_t start_stride_bh,
    size_t start_stride_seg, const float *__restrict__ start_z, size_t start_z_stride_bh, float *__restrict__ s_final,
    float *__restrict__ z_final, int N, int P, int seg_len, float eps, float *__restrict__ den_out,
    const float *__restrict__ start_vb) {
    constexpr int phi_mode = PHI;
    using TK = Tile<DK>;
    using TV = Tile<DV>;
    constexpr int KS = DK / 32;
    constexpr int NT = DV / 16;
    constexpr int NTO = NT / 2; // output tiles per wave
    __shared__ __attribute__((aligned(16))) uint16_t sQ[kChunk * TK::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * TK::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sKs[GATED ? kChunk * TK::RS : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kChunk * TV::RS];
    // S in bf16 (TileS, rows dk), and z in bf16 as one row that every lane of
    // the denominator tile reads (a broadcast), so that tile holds phi(q).z.
    __shared__ __attribute__((aligned(16))) uint16_t sS[DK * DV];
    __shared__ __attribute__((aligned(16))) uint16_t sZr[DK];
    // gated: the chunk's inclusive gate prefix per token, as kappa (decay_k)
    __shared__ __attribute__((aligned(16))) float sGk[GATED ? kChunk : 4];

    const int seg = blockIdx.x % P, bh = blockIdx.x / P;
    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int l16 = lane & 15, g = lane >> 4, qd = lane & 3;
    // Query block per wave: waves w and w + 4 share a SIMD, so blocks (0, 3) and
    // (1, 2) -- light and heavy ends of the causal triangle -- are paired.
    const int qblk_w = w < 4 ? (w >> 1) : 5 - (w >> 1), dh = w & 1;
    const bf16x8 ones = bf16_ones8();
    const int t_begin = seg * seg_len;
    const int t_end = min(N, t_begin + seg_len);
    const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
    const size_t row0 = (size_t)bh * N + t_begin;
    const uint16_t *qbp = q + row0 * DK;
    const uint16_t *kbp = k + row0 * DK;
    const uint16_t *vbp = v + row0 * DV;
    uint16_t *obp = o + row0 * DV;
    const float *ab = GATED ? alpha + row0 : nullptr;

    State8<DK, DV> st;
    {
        const float *s0 = start ? start + bh * start_stride_bh + seg * start_stride_seg : nullptr;
        const float *z0 = start_z ? start_z + bh * start_z_stride_bh + seg * start_stride_seg : nullptr;
        state8_load<DK, DV>(st, s0, z0, w, lane);
        if (TRAIN && start_vb) {
            using S8 = State8<DK, DV>;
            const float *vb0 = start_vb + bh * start_z_stride_bh + seg * start_stride_seg;
            const int nt0 = (w & 3) * S8::NTW;
#pragma unroll
            for (int mi = 0; mi < S8::MTW; ++mi) {
#pragma unroll
                for (int ni = 0; ni < S8::NTW; ++ni) {
                    const float4 vb = *reinterpret_cast<const float4 *>(vb0 + 16 * (nt0 + ni) + 4 * g);
                    st.s[mi][ni] += f32x4{vb.x, vb.y, vb.z, vb.w};
                }
            }
            if (S8::has_z(w)) st.z += (float)t_begin;
        }
        state8_z_to_lds<DK, DV>(st, sZr, w, lane);
    }
    state8_to_lds<DK, DV>(st, sS, w, lane);

    auto rows_in = [&](int c) { return min(kChunk, t_end - t_begin - c * kChunk); };

    // Q, K, V (and gates) are loaded two chunks ahead without gates and one
    // with them (where the decay bookkeeping needs the registers); each buffer
    // is refilled as soon as it is staged.
    constexpr int DEPTH = GATED ? 1 : 2;
    struct Buf {
        Units<DK> k;
        Units<DV> v;
        Units<DK> q;
        float a;
    };
    auto issue = [&](Buf &b, int c) {
        const int nv = rows_in(c);
        b.k.load(kbp + (size_t)c * kChunk * DK, nv, tid);
        b.v.load(vbp + (size_t)c * kChunk * DV, nv, tid);
        b.q.load(qbp + (size_t)c * kChunk * DK, nv, tid);
        if (GATED) b.a = lane < nv ? ab[c * kChunk + lane] : 1.f;
    };
    auto step = [&](Buf &b, int c) {
        const int valid = rows_in(c);
        // ---- stage: phi(Q), phi(K) (and decayed phi(K)), V, all row-major
        ChunkGates cg;
        float dC = 1.f, ke = 0.f;
        if (GATED) {
            cg.build(b.a, lane < valid);
            ke = cg.kappa_at(valid - 1);
            dC = decay_k(ke, 0.f);
            if (w == 0) sGk[lane] = cg.kappa();
        }
#pragma unroll
        for (int i = 0; i < Units<DK>::N; ++i) {
            const int row = Units<DK>::row_of(tid, i), col = Units<DK>::col_of(tid, i);
            *reinterpret_cast<uint4 *>(sQ + TK::off(row, col)) = phi_pack8(b.q.r[i], phi_mode);
            if (GATED) {
                const float sc = decay_k(ke, cg.kappa_at(row));
                uint4 plain, scaled;
                phi_pack8x2(b.k.r[i], phi_mode, sc, plain, scaled);
                *reinterpret_cast<uint4 *>(sK + TK::off(row, col)) = plain;
                *reinterpret_cast<uint4 *>(sKs + TK::off(row, col)) = scaled;
            } else {
                *reinterpret_cast<uint4 *>(sK + TK::off(row, col)) = phi_pack8(b.k.r[i], phi_mode);
            }
        }
#pragma unroll
        for (int i = 0; i < Units<DV>::N; ++i)
            *reinterpret_cast<uint4 *>(sV + TV::off(Units<DV>::row_of(tid, i), Units<DV>::col_of(tid, i))) =
                b.v.r[i];
        if (c + DEPTH < nch) issue(b, c + DEPTH);
        __syncthreads();
        // The chunk's matrix work is specialized on the wave's query block, so
        // the causal triangle (which key blocks are scored, which one is
        // masked) is fixed at compile time: no per-block branches and no
        // zero-filled skipped tiles.
        auto chunk_work = [&](auto qblk_c) {
            constexpr int qblk = decltype(qblk_c)::value;
            // ---- phi(Q) operands of this wave's query block
            bf16x8 qa[KS];
    #pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qa[ks] = *reinterpret_cast<const bf16x8 *>(sQ + TK::off(16 * qblk + l16, 32 * ks + 8 * g));

            // ---- scores A^T[key][query], key blocks 0..qblk
            f32x4 sc[4];
    #pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4) {
                sc[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (kb4 <= qblk) {
    #pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sK + TK::off(16 * kb4 + l16, 32 * ks + 8 * g));
                        sc[kb4] = mfma16x16x32(a, qa[ks], sc[kb4]);
                    }
                }
            }
            const int tq = 16 * qblk + l16;
            const float kq = GATED ? sGk[tq] : 0.f;
    #pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4) {
                if (kb4 <= qblk) {
                    float4 kk = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (GATED) kk = *reinterpret_cast<const float4 *>(sGk + 16 * kb4 + 4 * g);
                    const float kka[4] = {kk.x, kk.y, kk.z, kk.w};
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tk = 16 * kb4 + 4 * g + i;
                        float s = sc[kb4][i];
                        // the decay first: above the diagonal it may be inf, and
                        // the mask then replaces the product
                        if (GATED) s *= decay_k(kq, kka[i]);
                        if (kb4 == qblk && tk > tq) s = 0.f;
                        sc[kb4][i] = s;
                    }
                }
            }

            // ---- summary read: O^T = S^T phi(Q)^T for this wave's value columns
            // (S^T rows in the permuted value order, read transposed from S)
            f32x4 oacc[NTO];
    #pragma unroll
            for (int j = 0; j < NTO; ++j) {
                oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int nt = dh * NTO + j;
                const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
    #pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int klo = 32 * ks + 8 * g;
                    oacc[j] = mfma16x16x32(tr_operand_in<TileS<DV>>(sS, klo, klo + 4, colq, lane), qa[ks], oacc[j]);
                }
            }
            // denominator tile: every A row is z, so every element is phi(q).z
            f32x4 dt = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sZr + 32 * ks + 8 * g);
                dt = mfma16x16x32(a, qa[ks], dt);
            }
            if (GATED) {
                const float dq = decay_k(kq, 0.f);
                dt *= dq;
    #pragma unroll
                for (int j = 0; j < NTO; ++j) oacc[j] *= dq;
            }

            // ---- in-chunk part: O^T += V^T A^T (keys permuted within 32-key steps)
    #pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (2 * s2 <= qblk) {
                    uint4 bu;
                    bu.x = pack_bf16x2(sc[2 * s2][0], sc[2 * s2][1]);
                    bu.y = pack_bf16x2(sc[2 * s2][2], sc[2 * s2][3]);
                    bu.z = pack_bf16x2(sc[2 * s2 + 1][0], sc[2 * s2 + 1][1]);
                    bu.w = pack_bf16x2(sc[2 * s2 + 1][2], sc[2 * s2 + 1][3]);
                    const bf16x8 bop = as_bf16x8(bu);
                    // row sums of the scores into the denominator tile
                    dt = mfma16x16x32(ones, bop, dt);
                    const int klo = 32 * s2 + 4 * g, khi = klo + 16;
    #pragma unroll
                    for (int j = 0; j < NTO; ++j) {
                        const int nt = dh * NTO + j;
                        const int colq = 32 * (nt >> 1) + 8 * qd + 4 * (nt & 1);
                        oacc[j] = mfma16x16x32(tr_operand<DV>(sV, klo, khi, colq, lane), bop, oacc[j]);
                    }
                }
            }

            // ---- normalize and store: 16 rows x this wave's half of Dv
            if (tq < valid) {
                const float inv = __builtin_amdgcn_rcpf(dt[0] + eps); // 1 ulp; the result is rounded to bf16
                uint16_t *orow = obp + ((size_t)c * kChunk + tq) * DV;
                if (TRAIN && dh == 0 && g == 0) den_out[row0 + (size_t)c * kChunk + tq] = dt[0] + eps;
    #pragma unroll
                for (int pp = 0; pp < NTO / 2; ++pp) {
                    const int p = dh * (NTO / 2) + pp;
                    uint4 u;
                    u.x = pack_bf16x2(oacc[2 * pp][0] * inv, oacc[2 * pp][1] * inv);
                    u.y = pack_bf16x2(oacc[2 * pp][2] * inv, oacc[2 * pp][3] * inv);
                    u.z = pack_bf16x2(oacc[2 * pp + 1][0] * inv, oacc[2 * pp + 1][1] * inv);
                    u.w = pack_bf16x2(oacc[2 * pp + 1][2] * inv, oacc[2 * pp + 1][3] * inv);
                    *reinterpret_cast<uint4 *>(orow + 32 * p + 8 * g) = u;
                }
            }

        };
        switch (qblk_w) {
        case 0: chunk_work(std::integral_constant<int, 0>{}); break;
        case 1: chunk_work(std::integral_constant<int, 1>{}); break;
        case 2: chunk_work(std::integral_constant<int, 2>{}); break;
        default: chunk_work(std::integral_constant<int, 3>{}); break;
        }

        // ---- carry the state across the chunk, stage S (and z) for the next
        if (GATED) state8_scale<DK, DV>(st, dC);
        state8_update<DK, DV>(st, GATED ? sKs : sK, sV, w, lane, ones, phi_mode ? 0.f : (float)(kChunk - valid));
        __syncthreads();
        if (c + 1 < nch) {
            state8_z_to_lds<DK, DV>(st, sZr, w, lane);
            state8_to_lds<DK, DV>(st, sS, w, lane);
        }
    };

    if constexpr (DEPTH == 2) {
        Buf b0, b1;
        issue(b0, 0);
        if (nch > 1) issue(b1, 1);
        for (int c = 0; c < nch; c += 2) {
            step(b0, c);
            if (c + 1 < nch) step(b1, c + 1);
        }
    } else {
        Buf b0;
        issue(b0, 0);
        for (int c = 0; c < nch; ++c) step(b0, c);
    }
    if (s_final && seg == P - 1) {
        state8_store<DK, DV>(st, s_final + (size_t)bh * DK * DV, w, lane);
        state8_store_z<DK, DV>(st, z_final + (size_t)bh * DK, w, lane);
    }
}

} // namespace linattn
