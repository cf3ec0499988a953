// api.hip -- the C ABI of include/linattn.h: argument checks, the segment
// plan, kernel dispatch and the optional per-kernel timing.
#include <hip/hip_runtime.h>
#include <type_traits>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/linattn.h"
#include "fwd_bf16.hpp"
#include "fwd8_bf16.hpp"
#include "bwd8_bf16.hpp"
#include "delta8_bf16.hpp"
#include "recur.hpp"
#include "scan_decode.hpp"

using namespace linattn;

// Fixed device scratch of linattn_forward_noalloc (the segment states that
// linattn_forward keeps in the caller's workspace).  Each GPU the library runs
// on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel: its device address on the current GPU comes from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[LINATTN_NOALLOC_SCRATCH_BYTES];

namespace {

// ------------------------------------------------------------------ plan
// The sequence of each (b, h) is cut into P segments of seg_len tokens (a
// multiple of the 64-token chunk).  Segments run in parallel; the state each
// segment starts from is the prefix of the states of the segments before it.
// P is chosen so that P * B * H workgroups cover the 256 compute units.
constexpr int kTargetGroupsMfma = 256;      // output pass: one workgroup per compute unit
constexpr int kTargetGroupsState = 512;     // state pass: two per compute unit
constexpr int kTargetWavesRecur = 2048;

struct Plan {
    bool mfma = false;
    int P = 1;        // output segments per (b, h)
    int seg_len = 0;  // tokens per output segment
    int R = 1;        // state sub-segments per output segment
    int Ps = 1;       // state cells per (b, h): P * R (+ 1 for the forward kinds)
    int sub_len = 0;  // tokens per state sub-segment
    int nvb = 1;      // 64-column value blocks (recurrence path)
    size_t E = 0;     // floats of one state (Dk * Dv + Dk)
    size_t Eb = 0;    // backward: a forward state cell with the column sums of V (E + Dv)
    size_t ws_states = 0, ws_gam = 0, ws_total = 0, ws_rev = 0, ws_dd = 0, ws_bytes = 0;
};

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The prefix and suffix kernels address one (b, h)'s state cells through a
// buffer descriptor and drop unwanted stores by an offset of 1 GiB
// (kDropOffset): a split may not give one (b, h) 1 GiB of cells.  Only a
// caller-chosen split can come near this.
bool cells_fit(const Plan &p) { return (size_t)p.Ps * (p.Eb ? p.Eb : p.E) * sizeof(float) < (size_t(1) << 30); }

// seg_req, sub_req > 0 replace the automatic choice of the number of output
// segments and of state sub-segments per output segment (linattn_forward_planned):
// the sequence is cut into segments of ceil(chunks / seg_req) chunks (so at most
// seg_req of them), each into the largest divisor of its chunk count that does
// not exceed sub_req.
Plan make_plan(int kind, int B, int H, int N, int Dk, int Dv, int dtype, int seg_req = 0, int sub_req = 0) {
    Plan p;
    p.mfma = dtype == LINATTN_BF16 && Dk >= 32 && Dv >= 32;
    p.nvb = (Dv + 63) / 64;
    const long long BH = (long long)B * H;
    const int nch = (N + kChunk - 1) / kChunk;
    long long want = p.mfma ? (kTargetGroupsMfma + BH - 1) / BH : (kTargetWavesRecur + BH * p.nvb - 1) / (BH * p.nvb);
    if (seg_req > 0) want = seg_req;
    if (want < 1) want = 1;
    if (want > nch) want = nch;
    const int cps = (int)((nch + want - 1) / want);
    p.P = (nch + cps - 1) / cps;
    p.seg_len = cps * kChunk;
    // The state pass streams only K and V and fits two workgroups per compute
    // unit: split each output segment into R sub-segments (R divides cps).
    if (p.mfma) {
        long long want_r = (kTargetGroupsState + (long long)p.P * BH - 1) / ((long long)p.P * BH);
        if (sub_req > 0) want_r = sub_req;
        for (int r = (int)(want_r < cps ? want_r : cps); r >= 1; --r)
            if (cps % r == 0) {
                p.R = r;
                break;
            }
    }
    p.Ps = p.P * p.R;
    // the forward kinds keep one more cell per (b, h): the state at the end of
    // the sequence, which snapshots near the end are taken back from
    if ((kind == LINATTN_KIND_FORWARD || kind == LINATTN_KIND_GATED) && p.P > 1) p.Ps += 1;
    p.sub_len = p.seg_len / p.R;
    p.E = (size_t)Dk * Dv + Dk;
    p.Eb = p.E + Dv;
    const bool backward = kind == LINATTN_KIND_BACKWARD;
    const bool need_states = kind == LINATTN_KIND_NONCAUSAL || p.P > 1;
    // the backward keeps the forward's segment states (cells of Eb floats),
    // then the reverse sums of the later segments, then dd of every token; the
    // training forward's cells also carry the column sums of V (Eb floats)
    const bool wide = backward || kind == LINATTN_KIND_TRAIN;
    if (need_states) p.ws_states = align256((size_t)BH * p.Ps * (wide ? p.Eb : p.E) * sizeof(float));
    if (backward && p.P > 1) p.ws_rev = align256((size_t)BH * p.Ps * p.E * sizeof(float));
    if (backward) p.ws_dd = align256((size_t)BH * N * sizeof(float));
    if (kind == LINATTN_KIND_GATED && p.P > 1) p.ws_gam = align256((size_t)BH * p.Ps * sizeof(float));
    if (kind == LINATTN_KIND_NONCAUSAL) p.ws_total = align256((size_t)BH * p.E * sizeof(float));
    p.ws_bytes = p.ws_states + p.ws_gam + p.ws_total + p.ws_rev + p.ws_dd;
    return p;
}

// ------------------------------------------------------------------ timing
struct ProfRec {
    const char *name;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;      // recorded launches since enable
std::vector<hipEvent_t> g_events; // event pool, reused across enables
size_t g_event_next = 0;

hipEvent_t prof_event() {
    if (g_event_next == g_events.size()) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        g_events.push_back(e);
    }
    return g_events[g_event_next++];
}

// Set while linattn_forward_noalloc runs on this thread: its launches take
// no part in the timing record (which would create events).
thread_local bool t_noalloc = false;

// Launch helper: records an event pair around the launch while profiling.
template <typename F> int launch(const char *name, hipStream_t st, F &&fn) {
    ProfRec rec{name, nullptr, nullptr};
    const bool prof = g_prof_on && !t_noalloc;
    if (prof) {
        rec.a = prof_event();
        rec.b = prof_event();
        if (rec.a) hipEventRecord(rec.a, st);
    }
    fn();
    const hipError_t err = hipGetLastError();
    if (prof && rec.a && rec.b) {
        hipEventRecord(rec.b, st);
        g_prof.push_back(rec);
    }
    return err == hipSuccess ? LINATTN_OK : LINATTN_ELAUNCH;
}

#define LA_TRY(x)                                                                                                      \
    do {                                                                                                               \
        const int rc_ = (x);                                                                                           \
        if (rc_ != LINATTN_OK) return rc_;                                                                             \
    } while (0)

// ------------------------------------------------------------------ no-alloc scratch
// Device address of `scratch` on the GPU the stream belongs to, looked up once
// per device with that device current, and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(hipStream_t st, void **out) {
    int dev = -1;
    if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) return LINATTN_ELAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return LINATTN_ELAUNCH;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return LINATTN_ELAUNCH;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return LINATTN_ELAUNCH;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return LINATTN_ELAUNCH;
        if (e != hipSuccess || !p) return LINATTN_ELAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LINATTN_OK;
}

// ------------------------------------------------------------------ checks
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int check_common(int B, int H, int N, int Dk, int Dv, int dtype, int phi, float eps) {
    if (B < 1 || H < 1 || N < 1) return LINATTN_EINVAL;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return LINATTN_EINVAL;
    if (dtype != LINATTN_F32 && dtype != LINATTN_BF16) return LINATTN_EDTYPE;
    if (phi != LINATTN_PHI_ELU1 && phi != LINATTN_PHI_IDENTITY) return LINATTN_EDTYPE;
    if (!dim_ok(Dk) || !dim_ok(Dv)) return LINATTN_ESHAPE;
    // every index is formed in 64-bit; keep the element counts well inside it
    const long double elems = (long double)B * H * (long double)N * (Dk > Dv ? Dk : Dv);
    if (elems > 9.0e15L) return LINATTN_ESHAPE;
    if ((long long)B * H > 0x7fffffffLL / 64) return LINATTN_ESHAPE;
    return LINATTN_OK;
}

// ------------------------------------------------------------------ dispatch
// Head dims of 64 and 128 use the eight-wave kernels (fwd8_bf16.hpp); 32 uses
// the four-wave ones.
template <int DK, int DV> constexpr bool kEight = DK >= 64 && DV >= 64;

// Runs f(std::integral_constant<int, PHI>) for the feature map in use, for
// kernels that take it as a template parameter.
template <typename F> void with_phi(int phi, F &&f) {
    if (phi == LINATTN_PHI_IDENTITY)
        f(std::integral_constant<int, LINATTN_PHI_IDENTITY>{});
    else
        f(std::integral_constant<int, LINATTN_PHI_ELU1>{});
}

// Snapshot request of linattn_forward_snapshots (null: none).
struct SnapRequest {
    SnapList list;
    float *s_snap, *z_snap;
};
static_assert(kMaxSnapshots == LINATTN_MAX_SNAPSHOTS, "snapshot limit");

template <int DK, int DV, bool GATED>
int run_mfma_causal(const Plan &pl, const void *q, const void *k, const void *v, const float *alpha, void *o,
                    const float *s_init, const float *z_init, float *s_final, float *z_final, float *den,
                    const SnapRequest *snap, int BH, int N, int phi, float eps, char *ws, hipStream_t st) {
    const float *start = s_init, *start_z = z_init, *start_vb = nullptr;
    size_t sbh = (size_t)DK * DV, sseg = 0, zbh = DK;
    if (pl.P > 1) {
        float *states = reinterpret_cast<float *>(ws);
        float *gam = GATED ? reinterpret_cast<float *>(ws + pl.ws_states) : nullptr;
        // the training forward (den given) keeps its cells for the backward,
        // with the column sums of V appended (cells of Eb floats)
        const bool train = den != nullptr;
        const size_t E = train ? pl.Eb : pl.E;
        // the sub-segments of the last output segment are never needed by
        // the output pass; snapshots use them all, so that every snapshot lies
        // between two cells, the last one being the state at the end
        const int P_run = snap ? pl.P * pl.R : (pl.P - 1) * pl.R;
        LA_TRY(launch("seg_state_bf16", st, [&] {
            if constexpr (kEight<DK, DV>)
                with_phi(phi, [&](auto PH) {
                    if constexpr (!GATED) {
                        if (train) {
                            // the backward's form: for elu + 1, sums of elu(k) v^T
                            // and elu(k) (full relative precision in bf16) and of v
                            constexpr int FEAT = PH() == LINATTN_PHI_ELU1 ? kFeatElu : PH();
                            seg_state8_bf16<DK, DV, false, FEAT, true><<<dim3(P_run * BH), dim3(kThreads8), 0, st>>>(
                                (const uint16_t *)k, (const uint16_t *)v, alpha, states, gam, N, pl.Ps, P_run,
                                pl.sub_len);
                            return;
                        }
                    }
                    seg_state8_bf16<DK, DV, GATED, PH()><<<dim3(P_run * BH), dim3(kThreads8), 0, st>>>(
                        (const uint16_t *)k, (const uint16_t *)v, alpha, states, gam, N, pl.Ps, P_run, pl.sub_len);
                });
            else
                seg_state_bf16<DK, DV, GATED><<<dim3(P_run * BH), dim3(kThreads), 0, st>>>(
                    (const uint16_t *)k, (const uint16_t *)v, alpha, states, gam, N, pl.Ps, P_run, pl.sub_len, phi);
        }));
        // the output pass reads the cells at segment starts (every R-th);
        // snapshots may start from any cell
        LA_TRY(launch("seg_prefix", st, [&] {
            seg_prefix<<<dim3((unsigned)((E + 255) / 256), BH), dim3(256), 0, st>>>(
                states, gam, s_init, z_init, pl.Ps, P_run + 1, DK, DV, (int)E, snap ? 1 : pl.R);
        }));
        if (snap) {
            if constexpr (kEight<DK, DV>) {
                LA_TRY(launch("snap_state_bf16", st, [&] {
                    with_phi(phi, [&](auto PH) {
                        snap_state8_bf16<DK, DV, GATED, PH()><<<dim3(snap->list.n * BH), dim3(kThreads8), 0, st>>>(
                            (const uint16_t *)k, (const uint16_t *)v, alpha, states, (size_t)pl.Ps * pl.E,
                            pl.sub_len, P_run, nullptr, nullptr, snap->s_snap, snap->z_snap, N, snap->list);
                    });
                }));
            }
        }
        // output segment p starts from the prefix before state cell p * R
        start = states;
        start_z = states + (size_t)DK * DV;
        // training cells for elu + 1: E, zeta and the column sums of V
        if (train && phi == LINATTN_PHI_ELU1) start_vb = states + (size_t)DK * DV + DK;
        sbh = (size_t)pl.Ps * E;
        sseg = (size_t)pl.R * E;
        zbh = (size_t)pl.Ps * E;
    }
    if (snap && pl.P == 1) {
        // one segment: every snapshot runs from the initial state at token 0
        if constexpr (kEight<DK, DV>) {
            LA_TRY(launch("snap_state_bf16", st, [&] {
                with_phi(phi, [&](auto PH) {
                    snap_state8_bf16<DK, DV, GATED, PH()><<<dim3(snap->list.n * BH), dim3(kThreads8), 0, st>>>(
                        (const uint16_t *)k, (const uint16_t *)v, alpha, nullptr, 0, pl.seg_len, 0, s_init, z_init,
                        snap->s_snap, snap->z_snap, N, snap->list);
                });
            }));
        }
    }
    return launch(GATED ? "fwd_out_bf16_gated" : "fwd_out_bf16", st, [&] {
        if constexpr (kEight<DK, DV>)
            with_phi(phi, [&](auto PH) {
                // the training forward (den given, never gated) is its own instantiation
                if (den) {
                    if constexpr (!GATED)
                        fwd_out8_bf16<DK, DV, GATED, PH(), true><<<dim3(pl.P * BH), dim3(kThreads8), 0, st>>>(
                            (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, alpha, (uint16_t *)o,
                            start, sbh, sseg, start_z, zbh, s_final, z_final, N, pl.P, pl.seg_len, eps, den,
                            start_vb);
                } else
                    fwd_out8_bf16<DK, DV, GATED, PH()><<<dim3(pl.P * BH), dim3(kThreads8), 0, st>>>(
                        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, alpha, (uint16_t *)o, start,
                        sbh, sseg, start_z, zbh, s_final, z_final, N, pl.P, pl.seg_len, eps, nullptr, nullptr);
            });
        else
            fwd_out_bf16<DK, DV, GATED><<<dim3(pl.P * BH), dim3(kThreads), 0, st>>>(
                (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, alpha, (uint16_t *)o, start, sbh, sseg,
                start_z, zbh, s_final, z_final, N, pl.P, pl.seg_len, phi, eps);
    });
}

template <int DK, int DV>
int run_mfma_noncausal(const Plan &pl, const void *q, const void *k, const void *v, void *o, float *s_out,
                       float *z_out, int BH, int N, int phi, float eps, char *ws, hipStream_t st) {
    float *states = reinterpret_cast<float *>(ws);
    float *total = reinterpret_cast<float *>(ws + pl.ws_states + pl.ws_gam);
    LA_TRY(launch("seg_state_bf16", st, [&] {
        if constexpr (kEight<DK, DV>)
            with_phi(phi, [&](auto PH) {
                seg_state8_bf16<DK, DV, false, PH()><<<dim3(pl.Ps * BH), dim3(kThreads8), 0, st>>>(
                    (const uint16_t *)k, (const uint16_t *)v, nullptr, states, nullptr, N, pl.Ps, pl.Ps, pl.sub_len);
            });
        else
            seg_state_bf16<DK, DV, false><<<dim3(pl.Ps * BH), dim3(kThreads), 0, st>>>(
                (const uint16_t *)k, (const uint16_t *)v, nullptr, states, nullptr, N, pl.Ps, pl.Ps, pl.sub_len, phi);
    }));
    LA_TRY(launch("seg_total", st, [&] {
        seg_total<<<dim3((unsigned)((pl.E + 255) / 256), BH), dim3(256), 0, st>>>(states, total, s_out, z_out, pl.Ps,
                                                                                  DK, DV);
    }));
    const int nch = (N + kChunk - 1) / kChunk;
    const long long want_blocks = (2048 + BH - 1) / BH;
    int cpb = (int)((nch + want_blocks - 1) / want_blocks);
    if (cpb < 1) cpb = 1;
    const int blocks = (nch + cpb - 1) / cpb;
    return launch("noncausal_apply_bf16", st, [&] {
        with_phi(phi, [&](auto PH) {
            noncausal_apply_bf16<DK, DV, PH()><<<dim3(blocks * BH), dim3(kThreads), 0, st>>>(
                (const uint16_t *)q, (uint16_t *)o, total, N, blocks, cpb, eps);
        });
    });
}

// Backward (ungated, bf16, Dk and Dv in {64, 128}): the forward state at
// segment starts (for elu + 1 as sums of elu(k) v^T, elu(k) and v), dQ (and
// dd) forward in time, reverse segment sums, dK / dV backward in time.
template <int DK, int DV>
int run_mfma_backward(const Plan &pl, const void *q, const void *k, const void *v, const float *den,
                      const float *saved, const void *dout, void *dq, void *dk, void *dv, const float *s_init,
                      const float *z_init, int BH, int N, int phi, float eps, char *ws, hipStream_t st) {
    if constexpr (!kEight<DK, DV>) {
        return LINATTN_ESHAPE;
    } else {
        const uint16_t *q16 = (const uint16_t *)q, *k16 = (const uint16_t *)k, *v16 = (const uint16_t *)v;
        const uint16_t *g16 = (const uint16_t *)dout;
        float *dd = reinterpret_cast<float *>(ws + pl.ws_states + pl.ws_rev);
        const float *start = s_init, *start_z = z_init, *start_vb = nullptr;
        size_t sbh = (size_t)DK * DV, sseg = 0, zbh = DK;
        float *rev = nullptr;
        if (pl.P > 1) {
            const float *states = saved;
            rev = reinterpret_cast<float *>(ws + pl.ws_states);
            const int P_run = (pl.P - 1) * pl.R;
            if (!saved) {
                float *cells = reinterpret_cast<float *>(ws);
                LA_TRY(launch("seg_state_bf16", st, [&] {
                    with_phi(phi, [&](auto PH) {
                        constexpr int FEAT = PH() == LINATTN_PHI_ELU1 ? kFeatElu : PH();
                        seg_state8_bf16<DK, DV, false, FEAT, true><<<dim3(P_run * BH), dim3(kThreads8), 0, st>>>(
                            k16, v16, nullptr, cells, nullptr, N, pl.Ps, P_run, pl.sub_len);
                    });
                }));
                LA_TRY(launch("seg_prefix", st, [&] {
                    seg_prefix<<<dim3((unsigned)((pl.Eb + 255) / 256), BH), dim3(256), 0, st>>>(
                        cells, nullptr, s_init, z_init, pl.Ps, P_run + 1, DK, DV, (int)pl.Eb, pl.R);
                }));
                states = cells;
            }
            // else: the training forward's prefix cells, of the same plan and
            // in the same form (E, zeta, column sums of V)
            start = states;
            start_z = states + (size_t)DK * DV;
            start_vb = states + (size_t)DK * DV + DK;
            sbh = (size_t)pl.Ps * pl.Eb;
            sseg = (size_t)pl.R * pl.Eb;
            zbh = (size_t)pl.Ps * pl.Eb;
        }
        // dQ and dd; for P > 1 also the reverse sums of every output segment
        // past the first (cell j: segment j + 1), the granularity the dK/dV
        // pass starts from
        LA_TRY(launch("bwd_dq_bf16", st, [&] {
            with_phi(phi, [&](auto PH) {
                bwd_dq8_bf16<DK, DV, PH()><<<dim3(pl.P * BH), dim3(kThreads8), 0, st>>>(
                    q16, k16, v16, den, g16, (uint16_t *)dq, dd, start, sbh, sseg, start_z, zbh, start_vb, N, pl.P,
                    pl.seg_len, eps, rev, (size_t)pl.Ps * pl.E, 1, pl.seg_len / kChunk);
            });
        }));
        if (pl.P > 1) {
            const int cells = pl.P - 1;
            LA_TRY(launch("seg_suffix", st, [&] {
                seg_suffix<<<dim3((unsigned)((pl.E + 255) / 256), BH), dim3(256), 0, st>>>(rev, pl.Ps, cells,
                                                                                          (int)pl.E);
            }));
        }
        // output segment p < P - 1 starts (going backward) from the sum over
        // cells j >= p; the last segment starts from zero
        return launch("bwd_dkv_bf16", st, [&] {
            with_phi(phi, [&](auto PH) {
                bwd_dkv8_bf16<DK, DV, PH()><<<dim3(pl.P * BH), dim3(kThreads8), 0, st>>>(
                    q16, k16, v16, den, dd, g16, (uint16_t *)dk, (uint16_t *)dv, rev, (size_t)pl.Ps * pl.E,
                    pl.E, N, pl.P, pl.seg_len);
            });
        });
    }
}

template <int DK, int DV> struct MfmaBackward {
    template <typename... A> static int run(A &&...a) { return run_mfma_backward<DK, DV>(a...); }
};

template <typename T, int DK, bool GATED>
int run_recur_causal(const Plan &pl, const void *q, const void *k, const void *v, const float *alpha, void *o,
                     const float *s_init, const float *z_init, float *s_final, float *z_final, int BH, int N, int Dv,
                     int phi, float eps, char *ws, hipStream_t st) {
    const float *start = s_init, *start_z = z_init;
    size_t sbh = (size_t)DK * Dv, sseg = 0, zbh = DK;
    const size_t E = pl.E;
    if (pl.P > 1) {
        float *states = reinterpret_cast<float *>(ws);
        float *gam = GATED ? reinterpret_cast<float *>(ws + pl.ws_states) : nullptr;
        const int P_run = pl.P - 1;
        LA_TRY(launch("recur_state", st, [&] {
            recur_kernel<T, DK, GATED, RECUR_STATE><<<dim3(P_run * BH * pl.nvb), dim3(64), 0, st>>>(
                (const T *)q, (const T *)k, (const T *)v, alpha, nullptr, nullptr, 0, 0, nullptr, 0, states,
                states + (size_t)DK * Dv, (size_t)pl.P * E, E, (size_t)pl.P * E, gam, N, pl.P, P_run, pl.seg_len, Dv,
                phi, eps);
        }));
        LA_TRY(launch("seg_prefix", st, [&] {
            seg_prefix<<<dim3((unsigned)((E + 255) / 256), BH), dim3(256), 0, st>>>(states, gam, s_init, z_init, pl.P,
                                                                                    pl.P, DK, Dv, (int)E, 1);
        }));
        start = states;
        start_z = states + (size_t)DK * Dv;
        sbh = (size_t)pl.P * E;
        sseg = E;
        zbh = (size_t)pl.P * E;
    }
    return launch(GATED ? "recur_causal_gated" : "recur_causal", st, [&] {
        recur_kernel<T, DK, GATED, RECUR_CAUSAL><<<dim3(pl.P * BH * pl.nvb), dim3(64), 0, st>>>(
            (const T *)q, (const T *)k, (const T *)v, alpha, (T *)o, start, sbh, sseg, start_z, zbh, s_final, z_final,
            (size_t)DK * Dv, 0, (size_t)DK, nullptr, N, pl.P, pl.P, pl.seg_len, Dv, phi, eps);
    });
}

template <typename T, int DK>
int run_recur_noncausal(const Plan &pl, const void *q, const void *k, const void *v, void *o, float *s_out,
                        float *z_out, int BH, int N, int Dv, int phi, float eps, char *ws, hipStream_t st) {
    const size_t E = pl.E;
    float *states = reinterpret_cast<float *>(ws);
    float *total = reinterpret_cast<float *>(ws + pl.ws_states + pl.ws_gam);
    LA_TRY(launch("recur_state", st, [&] {
        recur_kernel<T, DK, false, RECUR_STATE><<<dim3(pl.P * BH * pl.nvb), dim3(64), 0, st>>>(
            (const T *)q, (const T *)k, (const T *)v, nullptr, nullptr, nullptr, 0, 0, nullptr, 0, states,
            states + (size_t)DK * Dv, (size_t)pl.P * E, E, (size_t)pl.P * E, nullptr, N, pl.P, pl.P, pl.seg_len, Dv,
            phi, eps);
    }));
    LA_TRY(launch("seg_total", st, [&] {
        seg_total<<<dim3((unsigned)((E + 255) / 256), BH), dim3(256), 0, st>>>(states, total, s_out, z_out, pl.P, DK,
                                                                              Dv);
    }));
    return launch("recur_apply", st, [&] {
        recur_kernel<T, DK, false, RECUR_APPLY><<<dim3(pl.P * BH * pl.nvb), dim3(64), 0, st>>>(
            (const T *)q, (const T *)k, (const T *)v, nullptr, (T *)o, total, E, 0, total + (size_t)DK * Dv, E,
            nullptr, nullptr, 0, 0, 0, nullptr, N, pl.P, pl.P, pl.seg_len, Dv, phi, eps);
    });
}

// Dispatch over the compiled (Dk, Dv) set.
template <template <int, int> class F, typename... A> int by_dims_mfma(int Dk, int Dv, A &&...a) {
#define LA_CASE(X, Y)                                                                                                  \
    if (Dk == X && Dv == Y) return F<X, Y>::run(a...);
    LA_CASE(32, 32) LA_CASE(32, 64) LA_CASE(32, 128)
    LA_CASE(64, 32) LA_CASE(64, 64) LA_CASE(64, 128)
    LA_CASE(128, 32) LA_CASE(128, 64) LA_CASE(128, 128)
#undef LA_CASE
    return LINATTN_ESHAPE;
}

template <bool GATED> struct MfmaCausal {
    template <int DK, int DV> struct F {
        template <typename... A> static int run(A &&...a) { return run_mfma_causal<DK, DV, GATED>(a...); }
    };
};
template <int DK, int DV> struct MfmaNoncausal {
    template <typename... A> static int run(A &&...a) { return run_mfma_noncausal<DK, DV>(a...); }
};

template <typename T, bool GATED, typename... A> int recur_causal_dk(int Dk, A &&...a) {
    switch (Dk) {
    case 16: return run_recur_causal<T, 16, GATED>(a...);
    case 32: return run_recur_causal<T, 32, GATED>(a...);
    case 64: return run_recur_causal<T, 64, GATED>(a...);
    case 128: return run_recur_causal<T, 128, GATED>(a...);
    }
    return LINATTN_ESHAPE;
}
template <typename T, typename... A> int recur_noncausal_dk(int Dk, A &&...a) {
    switch (Dk) {
    case 16: return run_recur_noncausal<T, 16>(a...);
    case 32: return run_recur_noncausal<T, 32>(a...);
    case 64: return run_recur_noncausal<T, 64>(a...);
    case 128: return run_recur_noncausal<T, 128>(a...);
    }
    return LINATTN_ESHAPE;
}

int forward_impl(bool gated, const void *q, const void *k, const void *v, const float *alpha, void *o,
                 const float *s_init, const float *z_init, float *s_final, float *z_final, int B, int H, int N,
                 int Dk, int Dv, int dtype, int phi, float eps, void *workspace, size_t workspace_bytes,
                 void *hip_stream, float *den = nullptr, const SnapRequest *snap = nullptr, int seg_req = 0,
                 int sub_req = 0, int kind = -1) {
    LA_TRY(check_common(B, H, N, Dk, Dv, dtype, phi, eps));
    if (!q || !k || !v || !o || (gated && !alpha)) return LINATTN_EINVAL;
    if ((s_init == nullptr) != (z_init == nullptr)) return LINATTN_EINVAL;
    if ((s_final == nullptr) != (z_final == nullptr)) return LINATTN_EINVAL;
    const size_t es = dtype == LINATTN_BF16 ? 2 : 4;
    const size_t nq = (size_t)B * H * N * Dk * es, nv = (size_t)B * H * N * Dv * es;
    if (overlaps(o, nv, q, nq) || overlaps(o, nv, k, nq) || overlaps(o, nv, v, nv)) return LINATTN_EINVAL;
    if (kind < 0) kind = gated ? LINATTN_KIND_GATED : LINATTN_KIND_FORWARD;
    const Plan pl = make_plan(kind, B, H, N, Dk, Dv, dtype, seg_req, sub_req);
    if (!cells_fit(pl)) return LINATTN_ESHAPE;
    if (pl.ws_bytes && (!workspace || workspace_bytes < pl.ws_bytes)) return LINATTN_EWORKSPACE;
    hipStream_t st = (hipStream_t)hip_stream;
    char *ws = (char *)workspace;
    const int BH = B * H;
    if (pl.mfma) {
        if (gated)
            return by_dims_mfma<MfmaCausal<true>::F>(Dk, Dv, pl, q, k, v, alpha, o, s_init, z_init, s_final, z_final,
                                                    den, snap, BH, N, phi, eps, ws, st);
        return by_dims_mfma<MfmaCausal<false>::F>(Dk, Dv, pl, q, k, v, alpha, o, s_init, z_init, s_final, z_final,
                                                 den, snap, BH, N, phi, eps, ws, st);
    }
    if (dtype == LINATTN_BF16) {
        if (gated)
            return recur_causal_dk<uint16_t, true>(Dk, pl, q, k, v, alpha, o, s_init, z_init, s_final, z_final, BH, N,
                                                   Dv, phi, eps, ws, st);
        return recur_causal_dk<uint16_t, false>(Dk, pl, q, k, v, alpha, o, s_init, z_init, s_final, z_final, BH, N,
                                                Dv, phi, eps, ws, st);
    }
    if (gated)
        return recur_causal_dk<float, true>(Dk, pl, q, k, v, alpha, o, s_init, z_init, s_final, z_final, BH, N, Dv,
                                            phi, eps, ws, st);
    return recur_causal_dk<float, false>(Dk, pl, q, k, v, alpha, o, s_init, z_init, s_final, z_final, BH, N, Dv, phi,
                                         eps, ws, st);
}

template <typename T, int DK, int DV, typename SS>
void launch_decode(const void *q, const void *k, const void *v, SS *s, SS *z, const float *alpha, void *o, int BH,
                   int phi, float eps, hipStream_t st) {
    // 512 threads (at Dk = Dv = 128: eight 16-byte state loads in flight per
    // thread), measured faster than 256 or 1024 with the state streamed from HBM
    decode_step_kernel<T, DK, DV, SS, 512><<<dim3(BH), dim3(512), 0, st>>>((const T *)q, (const T *)k, (const T *)v,
                                                                         s, z, alpha, (T *)o, phi, eps);
}

template <typename T, typename SS = float>
bool decode_dims(int Dk, int Dv, const void *q, const void *k, const void *v, SS *s, SS *z, const float *alpha,
                 void *o, int BH, int phi, float eps, hipStream_t st) {
#define LA_D(X, Y)                                                                                                     \
    if (Dk == X && Dv == Y) {                                                                                          \
        launch_decode<T, X, Y, SS>(q, k, v, s, z, alpha, o, BH, phi, eps, st);                                         \
        return true;                                                                                                   \
    }
    LA_D(16, 16) LA_D(16, 32) LA_D(16, 64) LA_D(16, 128)
    LA_D(32, 16) LA_D(32, 32) LA_D(32, 64) LA_D(32, 128)
    LA_D(64, 16) LA_D(64, 32) LA_D(64, 64) LA_D(64, 128)
    LA_D(128, 16) LA_D(128, 32) LA_D(128, 64) LA_D(128, 128)
#undef LA_D
    return false;
}

} // namespace

// ====================================================================== C ABI
extern "C" {

int linattn_forward(const void *q, const void *k, const void *v, void *o, const float *s_init, const float *z_init,
                    float *s_final, float *z_final, int B, int H, int N, int Dk, int Dv, int dtype, int phi,
                    float eps, void *workspace, size_t workspace_bytes, void *hip_stream) {
    return forward_impl(false, q, k, v, nullptr, o, s_init, z_init, s_final, z_final, B, H, N, Dk, Dv, dtype, phi,
                        eps, workspace, workspace_bytes, hip_stream);
}

int linattn_forward_gated(const void *q, const void *k, const void *v, const float *alpha, void *o,
                          const float *s_init, const float *z_init, float *s_final, float *z_final, int B, int H,
                          int N, int Dk, int Dv, int dtype, int phi, float eps, void *workspace,
                          size_t workspace_bytes, void *hip_stream) {
    return forward_impl(true, q, k, v, alpha, o, s_init, z_init, s_final, z_final, B, H, N, Dk, Dv, dtype, phi, eps,
                        workspace, workspace_bytes, hip_stream);
}

int linattn_forward_planned(const void *q, const void *k, const void *v, const float *alpha, void *o,
                            const float *s_init, const float *z_init, float *s_final, float *z_final, int B, int H,
                            int N, int Dk, int Dv, int dtype, int phi, float eps, int segments, int subsegments,
                            void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (segments < 1 || subsegments < 1) return LINATTN_EINVAL;
    return forward_impl(alpha != nullptr, q, k, v, alpha, o, s_init, z_init, s_final, z_final, B, H, N, Dk, Dv,
                        dtype, phi, eps, workspace, workspace_bytes, hip_stream, nullptr, nullptr, segments,
                        subsegments);
}

size_t linattn_workspace_size_planned(int kind, int B, int H, int N, int Dk, int Dv, int dtype, int segments,
                                      int subsegments) {
    if (kind != LINATTN_KIND_FORWARD && kind != LINATTN_KIND_GATED) return 0;
    if (segments < 1 || subsegments < 1) return 0;
    if (check_common(B, H, N, Dk, Dv, dtype, LINATTN_PHI_ELU1, 0.f) != LINATTN_OK) return 0;
    const Plan pl = make_plan(kind, B, H, N, Dk, Dv, dtype, segments, subsegments);
    return cells_fit(pl) ? pl.ws_bytes : 0;
}

int linattn_forward_noalloc(const void *q, const void *k, const void *v, void *o, const float *s_init,
                            const float *z_init, float *s_final, float *z_final, int B, int H, int N, int Dk, int Dv,
                            int dtype, int phi, float eps, void *hip_stream) {
    LA_TRY(check_common(B, H, N, Dk, Dv, dtype, phi, eps));
    if (!q || !k || !v || !o) return LINATTN_EINVAL;
    const Plan pl = make_plan(LINATTN_KIND_FORWARD, B, H, N, Dk, Dv, dtype);
    if (pl.ws_bytes > (size_t)LINATTN_NOALLOC_SCRATCH_BYTES) return LINATTN_EWORKSPACE;
    void *ws = nullptr;
    if (pl.ws_bytes) LA_TRY(noalloc_scratch((hipStream_t)hip_stream, &ws));
    // the segment states are written before they are read: nothing to clear
    t_noalloc = true;
    const int rc = forward_impl(false, q, k, v, nullptr, o, s_init, z_init, s_final, z_final, B, H, N, Dk, Dv, dtype,
                                phi, eps, ws, pl.ws_bytes ? (size_t)LINATTN_NOALLOC_SCRATCH_BYTES : 0, hip_stream);
    t_noalloc = false;
    return rc;
}

// The training forward and the backward run the chunked bf16 kernels only.
int check_train(int Dk, int Dv, int dtype) {
    if (dtype != LINATTN_BF16) return LINATTN_EDTYPE;
    if ((Dk != 64 && Dk != 128) || (Dv != 64 && Dv != 128)) return LINATTN_ESHAPE;
    return LINATTN_OK;
}

int linattn_forward_train(const void *q, const void *k, const void *v, void *o, float *den, const float *s_init,
                          const float *z_init, float *s_final, float *z_final, int B, int H, int N, int Dk, int Dv,
                          int dtype, int phi, float eps, void *workspace, size_t workspace_bytes,
                          void *hip_stream) {
    LA_TRY(check_common(B, H, N, Dk, Dv, dtype, phi, eps));
    LA_TRY(check_train(Dk, Dv, dtype));
    if (!o || !den) return LINATTN_EINVAL;
    const size_t nq = (size_t)B * H * N * Dk * 2, nv = (size_t)B * H * N * Dv * 2, nd = (size_t)B * H * N * 4;
    if (overlaps(den, nd, q, nq) || overlaps(den, nd, k, nq) || overlaps(den, nd, v, nv) || overlaps(den, nd, o, nv))
        return LINATTN_EINVAL;
    return forward_impl(false, q, k, v, nullptr, o, s_init, z_init, s_final, z_final, B, H, N, Dk, Dv, dtype, phi,
                        eps, workspace, workspace_bytes, hip_stream, den, nullptr, 0, 0, LINATTN_KIND_TRAIN);
}

int linattn_forward_delta(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                          void *o, const float *s_init, float *s_final, int B, int H, int N, int Dk, int Dv,
                          int dtype, int phi, void *hip_stream) {
    LA_TRY(check_common(B, H, N, Dk, Dv, dtype, phi, 0.f));
    LA_TRY(check_train(Dk, Dv, dtype));
    if (!q || !k || !v || !o) return LINATTN_EINVAL;
    const size_t BH = (size_t)B * H;
    const size_t nq = BH * N * Dk * 2, nv = BH * N * Dv * 2, ns = BH * Dk * Dv * 4;
    const void *ins[6] = {q, k, v, beta, alpha, s_init};
    const size_t insz[6] = {nq, nq, nv, BH * N * 4, BH * N * 4, ns};
    for (int b = 0; b < 6; ++b)
        if (overlaps(o, nv, ins[b], insz[b]) || (b < 5 && overlaps(s_final, ns, ins[b], insz[b])))
            return LINATTN_EINVAL;
    if (overlaps(o, nv, s_final, ns)) return LINATTN_EINVAL;
    hipStream_t st = (hipStream_t)hip_stream;
    auto run = [&](auto DKc, auto DVc) {
        constexpr int DK = decltype(DKc)::value, DV = decltype(DVc)::value;
        return launch("delta_bf16", st, [&] {
            with_phi(phi, [&](auto PH) {
                auto go = [&](auto BT, auto GT) {
                    // Dv = 128: one wave per 16 value columns, each carrying its
                    // columns through the chunk in its own registers
                    if constexpr (DV == 128)
                        delta8c_bf16<DK, PH(), BT(), GT()><<<dim3((unsigned)BH), dim3(kThreads8), 0, st>>>(
                            (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, alpha, beta,
                            (uint16_t *)o, s_init, s_final, N);
                    else
                        delta8_bf16<DK, DV, PH(), BT(), GT()><<<dim3((unsigned)BH), dim3(kThreads8), 0, st>>>(
                            (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, alpha, beta,
                            (uint16_t *)o, s_init, s_final, N);
                };
                using T = std::true_type;
                using F = std::false_type;
                if (alpha) {
                    if (beta) go(T{}, T{});
                    else go(F{}, T{});
                } else {
                    if (beta) go(T{}, F{});
                    else go(F{}, F{});
                }
            });
        });
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    if (Dk == 64) return Dv == 64 ? run(I64{}, I64{}) : run(I64{}, I128{});
    return Dv == 64 ? run(I128{}, I64{}) : run(I128{}, I128{});
}

int linattn_forward_snapshots(const void *q, const void *k, const void *v, const float *alpha, void *o,
                              const float *s_init, const float *z_init, float *s_final, float *z_final,
                              const int *positions, int n_pos, float *s_snap, float *z_snap, int B, int H, int N,
                              int Dk, int Dv, int dtype, int phi, float eps, void *workspace, size_t workspace_bytes,
                              void *hip_stream) {
    LA_TRY(check_common(B, H, N, Dk, Dv, dtype, phi, eps));
    LA_TRY(check_train(Dk, Dv, dtype));
    if (!positions || !s_snap || !z_snap || n_pos < 1 || n_pos > LINATTN_MAX_SNAPSHOTS) return LINATTN_EINVAL;
    SnapRequest req;
    req.list.n = n_pos;
    for (int i = 0; i < n_pos; ++i) {
        if (positions[i] < 0 || positions[i] >= N) return LINATTN_EINVAL;
        req.list.pos[i] = positions[i];
    }
    for (int i = n_pos; i < kMaxSnapshots; ++i) req.list.pos[i] = 0;
    req.s_snap = s_snap;
    req.z_snap = z_snap;
    const size_t BH = (size_t)B * H;
    const size_t nq = BH * N * Dk * 2, nv = BH * N * Dv * 2, ns = BH * n_pos * Dk * Dv * 4, nz = BH * n_pos * Dk * 4;
    const void *others[7] = {q, k, v, o, alpha, s_final, z_final};
    const size_t osz[7] = {nq, nq, nv, nv, BH * N * 4, BH * Dk * Dv * 4, BH * Dk * 4};
    for (int b = 0; b < 7; ++b)
        if (overlaps(s_snap, ns, others[b], osz[b]) || overlaps(z_snap, nz, others[b], osz[b])) return LINATTN_EINVAL;
    if (overlaps(s_snap, ns, z_snap, nz)) return LINATTN_EINVAL;
    return forward_impl(alpha != nullptr, q, k, v, alpha, o, s_init, z_init, s_final, z_final, B, H, N, Dk, Dv,
                        dtype, phi, eps, workspace, workspace_bytes, hip_stream, nullptr, &req);
}

int linattn_backward(const void *q, const void *k, const void *v, const float *den, const void *saved,
                     const void *dout, void *dq, void *dk, void *dv, const float *s_init, const float *z_init, int B,
                     int H, int N, int Dk, int Dv, int dtype, int phi, float eps, void *workspace,
                     size_t workspace_bytes, void *hip_stream) {
    LA_TRY(check_common(B, H, N, Dk, Dv, dtype, phi, eps));
    LA_TRY(check_train(Dk, Dv, dtype));
    if (!q || !k || !v || !den || !dout || !dq || !dk || !dv) return LINATTN_EINVAL;
    if ((s_init == nullptr) != (z_init == nullptr)) return LINATTN_EINVAL;
    const size_t nq = (size_t)B * H * N * Dk * 2, nv = (size_t)B * H * N * Dv * 2, nd = (size_t)B * H * N * 4;
    const size_t ns = make_plan(LINATTN_KIND_TRAIN, B, H, N, Dk, Dv, dtype).ws_bytes;
    const void *ins[6] = {q, k, v, den, dout, saved};
    const size_t insz[6] = {nq, nq, nv, nd, nv, ns};
    void *outs[3] = {dq, dk, dv};
    const size_t outsz[3] = {nq, nq, nv};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlaps(outs[a], outsz[a], ins[b], insz[b])) return LINATTN_EINVAL;
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], outsz[a], outs[b], outsz[b])) return LINATTN_EINVAL;
    }
    const Plan pl = make_plan(LINATTN_KIND_BACKWARD, B, H, N, Dk, Dv, dtype);
    if (!workspace || workspace_bytes < pl.ws_bytes) return LINATTN_EWORKSPACE;
    if (overlaps(workspace, workspace_bytes, saved, ns)) return LINATTN_EINVAL;
    return by_dims_mfma<MfmaBackward>(Dk, Dv, pl, q, k, v, den, (const float *)saved, dout, dq, dk, dv, s_init,
                                      z_init, B * H, N, phi, eps, (char *)workspace, (hipStream_t)hip_stream);
}

int linattn_forward_noncausal(const void *q, const void *k, const void *v, void *o, float *s_out, float *z_out,
                              int B, int H, int N, int Dk, int Dv, int dtype, int phi, float eps, void *workspace,
                              size_t workspace_bytes, void *hip_stream) {
    LA_TRY(check_common(B, H, N, Dk, Dv, dtype, phi, eps));
    if (!q || !k || !v || !o) return LINATTN_EINVAL;
    if ((s_out == nullptr) != (z_out == nullptr)) return LINATTN_EINVAL;
    const size_t es = dtype == LINATTN_BF16 ? 2 : 4;
    const size_t nq = (size_t)B * H * N * Dk * es, nv = (size_t)B * H * N * Dv * es;
    if (overlaps(o, nv, q, nq) || overlaps(o, nv, k, nq) || overlaps(o, nv, v, nv)) return LINATTN_EINVAL;
    const Plan pl = make_plan(LINATTN_KIND_NONCAUSAL, B, H, N, Dk, Dv, dtype);
    if (!workspace || workspace_bytes < pl.ws_bytes) return LINATTN_EWORKSPACE;
    hipStream_t st = (hipStream_t)hip_stream;
    char *ws = (char *)workspace;
    const int BH = B * H;
    if (pl.mfma) return by_dims_mfma<MfmaNoncausal>(Dk, Dv, pl, q, k, v, o, s_out, z_out, BH, N, phi, eps, ws, st);
    if (dtype == LINATTN_BF16)
        return recur_noncausal_dk<uint16_t>(Dk, pl, q, k, v, o, s_out, z_out, BH, N, Dv, phi, eps, ws, st);
    return recur_noncausal_dk<float>(Dk, pl, q, k, v, o, s_out, z_out, BH, N, Dv, phi, eps, ws, st);
}

int linattn_decode_step(const void *q, const void *k, const void *v, float *s, float *z, const float *alpha,
                        void *o, int B, int H, int Dk, int Dv, int dtype, int phi, float eps, void *hip_stream) {
    LA_TRY(check_common(B, H, 1, Dk, Dv, dtype, phi, eps));
    if (!q || !k || !v || !s || !z || !o) return LINATTN_EINVAL;
    const size_t BH = (size_t)B * H;
    const size_t es = dtype == LINATTN_BF16 ? 2 : 4;
    if (overlaps(o, BH * Dv * es, s, BH * Dk * Dv * 4) || overlaps(o, BH * Dv * es, z, BH * Dk * 4) ||
        overlaps(s, BH * Dk * Dv * 4, z, BH * Dk * 4))
        return LINATTN_EINVAL;
    hipStream_t st = (hipStream_t)hip_stream;
    return launch("decode_step", st, [&] {
        if (dtype == LINATTN_BF16)
            decode_dims<uint16_t>(Dk, Dv, q, k, v, s, z, alpha, o, (int)BH, phi, eps, st);
        else
            decode_dims<float>(Dk, Dv, q, k, v, s, z, alpha, o, (int)BH, phi, eps, st);
    });
}

int linattn_decode_step_lowp(const void *q, const void *k, const void *v, void *s, void *z, int state_dtype,
                             const float *alpha, void *o, int B, int H, int Dk, int Dv, int dtype, int phi, float eps,
                             void *hip_stream) {
    LA_TRY(check_common(B, H, 1, Dk, Dv, dtype, phi, eps));
    if (state_dtype != LINATTN_F32 && state_dtype != LINATTN_BF16 && state_dtype != LINATTN_FP8_E4M3)
        return LINATTN_EDTYPE;
    if (!q || !k || !v || !s || !z || !o) return LINATTN_EINVAL;
    const size_t BH = (size_t)B * H;
    const size_t es = dtype == LINATTN_BF16 ? 2 : 4;
    const size_t ss = state_dtype == LINATTN_F32 ? 4 : state_dtype == LINATTN_BF16 ? 2 : 1;
    if (overlaps(o, BH * Dv * es, s, BH * Dk * Dv * ss) || overlaps(o, BH * Dv * es, z, BH * Dk * ss) ||
        overlaps(s, BH * Dk * Dv * ss, z, BH * Dk * ss))
        return LINATTN_EINVAL;
    hipStream_t st = (hipStream_t)hip_stream;
    auto go = [&](auto tq, auto ts) {
        using T = decltype(tq);
        using SS = decltype(ts);
        decode_dims<T, SS>(Dk, Dv, q, k, v, (SS *)s, (SS *)z, alpha, o, (int)BH, phi, eps, st);
    };
    return launch("decode_step", st, [&] {
        if (dtype == LINATTN_BF16) {
            if (state_dtype == LINATTN_F32) go(uint16_t{}, float{});
            else if (state_dtype == LINATTN_BF16) go(uint16_t{}, uint16_t{});
            else go(uint16_t{}, uint8_t{});
        } else {
            if (state_dtype == LINATTN_F32) go(float{}, float{});
            else if (state_dtype == LINATTN_BF16) go(float{}, uint16_t{});
            else go(float{}, uint8_t{});
        }
    });
}

size_t linattn_workspace_size(int kind, int B, int H, int N, int Dk, int Dv, int dtype) {
    if (kind < LINATTN_KIND_FORWARD || kind > LINATTN_KIND_TRAIN) return 0;
    if (check_common(B, H, N, Dk, Dv, dtype, LINATTN_PHI_ELU1, 0.f) != LINATTN_OK) return 0;
    return make_plan(kind, B, H, N, Dk, Dv, dtype).ws_bytes;
}

const char *linattn_status_string(int status) {
    switch (status) {
    case LINATTN_OK: return "ok";
    case LINATTN_EINVAL: return "invalid argument";
    case LINATTN_ESHAPE: return "unsupported shape";
    case LINATTN_EDTYPE: return "unsupported dtype or feature map";
    case LINATTN_EWORKSPACE: return "workspace too small";
    case LINATTN_ELAUNCH: return "HIP launch failed";
    }
    return "unknown status";
}

int linattn_abi_version(void) { return LINATTN_ABI_VERSION; }

int linattn_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (on) {
        g_prof.clear();
        g_event_next = 0;
    }
    g_prof_on = on != 0;
    return LINATTN_OK;
}

int linattn_profile_read(const char **names, double *total_ms, int *launches, int max) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    std::vector<const char *> nm;
    std::vector<double> ms;
    std::vector<int> cnt;
    for (const ProfRec &r : g_prof) {
        if (hipEventSynchronize(r.b) != hipSuccess) return LINATTN_ELAUNCH;
        float t = 0.f;
        if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return LINATTN_ELAUNCH;
        size_t i = 0;
        while (i < nm.size() && std::strcmp(nm[i], r.name) != 0) ++i;
        if (i == nm.size()) {
            nm.push_back(r.name);
            ms.push_back(0.0);
            cnt.push_back(0);
        }
        ms[i] += t;
        cnt[i] += 1;
    }
    for (size_t i = 0; i < nm.size() && (int)i < max; ++i) {
        if (names) names[i] = nm[i];
        if (total_ms) total_ms[i] = ms[i];
        if (launches) launches[i] = cnt[i];
    }
    return (int)nm.size();
}

} // extern "C"
