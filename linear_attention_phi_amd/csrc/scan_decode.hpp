// scan_decode.hpp -- segment-state prefix, non-causal total, and the
// one-token decode step.
#pragma once

#include "common.hpp"

namespace linattn {

// Cells whose loads the prefix and suffix kernels issue before their adds
// (8 and 16 measured alike, 32 slower).
constexpr int kCellBatch = 8;

// Exclusive prefix over the segments of each (b, h), in place:
//   ws[p] <- S_{<p} = a-decayed sum of the states of segments 0..p-1, seeded
//   with the caller's initial state (or zero).
// Summing the per-segment contributions is the associativity of the sum of
// outer products ("Linear Attention: accumulating KV into a fixed-size state",
// section "Adding to the same state in turn"); with gates, S_{<p+1} =
// G_p S_{<p} + dS_p where G_p is the product of segment p's gates.
// The order over segments is fixed, so the result is bitwise reproducible.
// Grid: x = element blocks of 256, y = bh.
// Cells 0..cells-2 hold segment states on entry; cells p = 0, every, 2 every,
// ... (and the last, cells - 1) receive the prefix (cell p gets the state
// before segment p); the others are left as they were.  P is the number of
// cells per (b, h); a cell is E floats (S, z, then any further sums, which
// start from zero).
__global__ __launch_bounds__(256) void seg_prefix(float *__restrict__ ws, const float *__restrict__ gam,
                                                  const float *__restrict__ s_init, const float *__restrict__ z_init,
                                                  int P, int cells, int DK, int DV, int E, int every) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int bh = blockIdx.y;
    if (e >= E) return;
    float run = 0.f;
    if (s_init && e < DK * DV + DK)
        run = e < DK * DV ? s_init[(size_t)bh * DK * DV + e] : z_init[(size_t)bh * DK + (e - DK * DV)];
    float *cell = ws + (size_t)bh * P * E + e;
    // The loop is a chain of dependent adds: kBatch segments' loads are issued
    // before any of their adds, so a chain of n cells waits ceil(n / kBatch)
    // memory latencies.  Loads and stores go through buffer descriptors over
    // this (b, h)'s cells, with no branch around them: a load past the
    // segment states reads 0, a store that is not wanted takes an offset past
    // the end and is dropped.
    constexpr int kBatch = kCellBatch;
    const rsrc_t rc = chunk_rsrc(ws + (size_t)bh * P * E, (cells - 1) * E * 4);
    const rsrc_t rw = chunk_rsrc(ws + (size_t)bh * P * E, cells * E * 4);
    const rsrc_t rg = chunk_rsrc(gam ? gam + (size_t)bh * P : ws, gam ? (cells - 1) * 4 : 0);
    for (int p0 = 0; p0 + 1 < cells; p0 += kBatch) {
        float d[kBatch], gm[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            d[j] = buffer_load_f32(rc, ((p0 + j) * E + e) * 4);
            if (gam) gm[j] = buffer_load_f32(rg, (p0 + j) * 4);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int p = p0 + j;
            // cells past the last segment state: d = 0 and a gate of 1 leave run as it is
            const bool in = p + 1 < cells;
            buffer_store_f32(run, rw, in && p % every == 0 ? (p * E + e) * 4 : kDropOffset);
            run = gam ? fmaf(in ? gm[j] : 1.f, run, d[j]) : run + d[j];
        }
    }
    cell[(size_t)(cells - 1) * E] = run;
}

// Inclusive suffix over the cells of each (b, h), in place and in a fixed
// order: cell j <- sum_{j' >= j} cell j' (the backward's sums over later
// segments).  P cells of E floats per (b, h).
__global__ __launch_bounds__(256) void seg_suffix(float *__restrict__ ws, int P, int cells, int E) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int bh = blockIdx.y;
    if (e >= E) return;
    float run = 0.f;
    // as in seg_prefix: kBatch loads ahead of their adds, no branch around a
    // load or a store (loads before the first cell read 0)
    constexpr int kBatch = kCellBatch;
    const rsrc_t rc = chunk_rsrc(ws + (size_t)bh * P * E, cells * E * 4);
    for (int j1 = cells; j1 > 0; j1 -= kBatch) {
        float d[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int j = j1 - 1 - i;
            d[i] = buffer_load_f32(rc, j >= 0 ? (j * E + e) * 4 : kDropOffset);
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            run += d[i];
            const int j = j1 - 1 - i;
            buffer_store_f32(run, rc, j >= 0 ? (j * E + e) * 4 : kDropOffset);
        }
    }
}

// Non-causal total: S = sum over all segments (fixed order), written to
// total[bh] and, when requested, to the caller's s_out / z_out.
__global__ __launch_bounds__(256) void seg_total(const float *__restrict__ ws, float *__restrict__ total,
                                                 float *__restrict__ s_out, float *__restrict__ z_out, int P, int DK,
                                                 int DV) {
    const int E = DK * DV + DK;
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int bh = blockIdx.y;
    if (e >= E) return;
    const float *cell = ws + (size_t)bh * P * E + e;
    float run = 0.f;
#pragma unroll 8
    for (int p = 0; p < P; ++p) run += cell[(size_t)p * E];
    total[(size_t)bh * E + e] = run;
    if (s_out) {
        if (e < DK * DV)
            s_out[(size_t)bh * DK * DV + e] = run;
        else
            z_out[(size_t)bh * DK + (e - DK * DV)] = run;
    }
}

template <typename T> __device__ __forceinline__ float load_elem(const T *p, size_t i);
template <> __device__ __forceinline__ float load_elem<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}
template <typename T> __device__ __forceinline__ void store_elem(T *p, size_t i, float v);
template <> __device__ __forceinline__ void store_elem<float>(float *p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_elem<uint16_t>(uint16_t *p, size_t i, float v) {
    p[i] = (uint16_t)f32_to_bf16_bits(v);
}

// Storage of the carried state: fp32, bf16 or fp8 (OCP e4m3, as converted by
// gfx950: round to nearest even, magnitudes past 448 become NaN).  Four
// consecutive elements at a time; rnd() is the value as stored.
template <typename SS> struct StateIO;
template <> struct StateIO<float> {
    __device__ static __forceinline__ f32x4 load4(const float *p, size_t u) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + u);
    }
    __device__ static __forceinline__ void store4(float *p, size_t u, f32x4 x) {
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p) + u);
    }
    __device__ static __forceinline__ float rnd(float x) { return x; }
    __device__ static __forceinline__ float load1(const float *p, size_t i) { return p[i]; }
    __device__ static __forceinline__ void store1(float *p, size_t i, float x) { p[i] = x; }
};
template <> struct StateIO<uint16_t> {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __device__ static __forceinline__ f32x4 load4(const uint16_t *p, size_t u) {
        const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p) + u);
        return f32x4{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
    }
    __device__ static __forceinline__ void store4(uint16_t *p, size_t u, f32x4 x) {
        const u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p) + u);
    }
    __device__ static __forceinline__ float rnd(float x) { return bf16_round(x); }
    __device__ static __forceinline__ float load1(const uint16_t *p, size_t i) { return bf16_bits_to_f32(p[i]); }
    __device__ static __forceinline__ void store1(uint16_t *p, size_t i, float x) {
        p[i] = (uint16_t)f32_to_bf16_bits(x);
    }
};
template <> struct StateIO<uint8_t> {
    __device__ static __forceinline__ f32x4 load4(const uint8_t *p, size_t u) {
        const int w = (int)__builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p) + u);
        return f32x4{__builtin_amdgcn_cvt_f32_fp8(w, 0), __builtin_amdgcn_cvt_f32_fp8(w, 1),
                     __builtin_amdgcn_cvt_f32_fp8(w, 2), __builtin_amdgcn_cvt_f32_fp8(w, 3)};
    }
    __device__ static __forceinline__ void store4(uint8_t *p, size_t u, f32x4 x) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
        __builtin_nontemporal_store((uint32_t)w, reinterpret_cast<uint32_t *>(p) + u);
    }
    __device__ static __forceinline__ float rnd(float x) {
        return __builtin_amdgcn_cvt_f32_fp8(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false), 0);
    }
    __device__ static __forceinline__ float load1(const uint8_t *p, size_t i) {
        return __builtin_amdgcn_cvt_f32_fp8((int)p[i], 0);
    }
    __device__ static __forceinline__ void store1(uint8_t *p, size_t i, float x) {
        p[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xff);
    }
};

// One decode step per (b, h), in place, streaming the state once:
//   S <- a S + phi(k) v^T,  z <- a z + phi(k),  o = phi(q)^T S / (phi(q)^T z + eps)
// (the read uses the updated state: "Linear Attention: accumulating KV into a
// fixed-size state", section "State update and read as equations"; the
// one-token-at-a-time RNN mode of the "Transformers are RNNs" review).
// SS is the storage type of S and z (fp32 normally; bf16 or fp8 to study the
// drift of a low-precision summary rewritten every token, which the
// product-order page warns about in "What a summary can't do"): the update is
// computed in fp32 from the stored values, rounded once to SS, and the read
// uses the value as stored.
// One workgroup of NT threads (NT >= Dk, Dv) per (b, h).  Thread -> (row group, 4-element
// column unit): the DV/4 units of a row are covered by consecutive threads,
// so every pass of the workgroup reads and writes whole rows (coalesced), and
// all passes are issued before any is consumed.
template <typename T, int DK, int DV, typename SS = float, int NT = 256>
__global__ __launch_bounds__(NT) void decode_step_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                          const T *__restrict__ v, SS *__restrict__ s,
                                                          SS *__restrict__ z, const float *__restrict__ alpha,
                                                          T *__restrict__ o, int phi_mode, float eps) {
    using IO = StateIO<SS>;
    constexpr int C4 = DV / 4;                 // float4 columns per row
    constexpr int RPP = NT / C4;               // rows one pass of the workgroup covers
    constexpr int ROWS = DK < RPP ? DK : RPP;  // rows per pass actually used
    constexpr int PASSES = DK / ROWS;
    constexpr int ACTIVE = ROWS * C4;          // threads holding state
    __shared__ float sq[DK], sk[DK], sv[DV];
    __shared__ __attribute__((aligned(16))) float red[ROWS][DV];
    constexpr int NW = NT / 64;
    __shared__ float sden[NW];

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const float a = alpha ? alpha[bh] : 1.f;
    SS *sb = s + (size_t)bh * DK * DV;
    const int c4 = tid % C4, r0 = tid / C4;
    const bool act = tid < ACTIVE;
    f32x4 st[PASSES];
    if (act) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) st[p] = IO::load4(sb, (size_t)(r0 + p * ROWS) * C4 + c4);
    }
    if (tid < DK) {
        sq[tid] = phi_exact(load_elem<T>(q, (size_t)bh * DK + tid), phi_mode);
        sk[tid] = phi_exact(load_elem<T>(k, (size_t)bh * DK + tid), phi_mode);
    }
    if (tid < DV) sv[tid] = load_elem<T>(v, (size_t)bh * DV + tid);
    __syncthreads();

    // z <- a z + phi(k) and the denominator phi(q).z (threads 0..DK-1)
    float dpart = 0.f;
    if (tid < DK) {
        const float zn = IO::rnd(fmaf(a, IO::load1(z, (size_t)bh * DK + tid), sk[tid]));
        IO::store1(z, (size_t)bh * DK + tid, zn);
        dpart = sq[tid] * zn;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dpart += __shfl_xor(dpart, m, 64);
    if ((tid & 63) == 0) sden[tid >> 6] = dpart;

    if (act) {
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
        const f32x4 vv = {sv[4 * c4], sv[4 * c4 + 1], sv[4 * c4 + 2], sv[4 * c4 + 3]};
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int row = r0 + p * ROWS;
            const float fk = sk[row], fq = sq[row];
            f32x4 x = st[p];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = IO::rnd(fmaf(a, x[e], fk * vv[e]));
                num[e] = fmaf(fq, x[e], num[e]);
            }
            IO::store4(sb, (size_t)row * C4 + c4, x);
        }
        *reinterpret_cast<f32x4 *>(&red[r0][4 * c4]) = num;
    }
    __syncthreads();
    if (tid < DV) {
        float acc = 0.f;
#pragma unroll 8
        for (int r = 0; r < ROWS; ++r) acc += red[r][tid];
        float den = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) den += sden[i];
        store_elem<T>(o, (size_t)bh * DV + tid, acc / (den + eps));
    }
}

} // namespace linattn
