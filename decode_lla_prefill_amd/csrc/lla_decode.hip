// lla_decode.hip -- the decode step and the state fill for gfx950 (MI355X).
//
// Decode (slide deck "Chunking, causality, and parallel prefill", "Mechanism
// map", decode line, and the instructor note answering the prefill/decode
// check): one token gives a 1x1 triangle, so all that is left is the rank-1
// state update and the state read,
//     S <- S + k v^T,      o = S^T q      (o[j] = sum_i q[i] S[i][j]).
//
// The step is bound by HBM: each (b,h) state of dk x dv fp32 is read once and
// written once, while q, k, v and o are a few hundred bytes.  One workgroup
// owns one (b,h).  A thread owns VW consecutive value columns and a strided
// set of key rows; all of its state rows are loaded before any is used (deep
// memory-level parallelism), each 16-byte row piece is updated in registers,
// written back with a streaming store, and folded into the thread's partial
// o; the partials of the row groups are summed through LDS in a fixed order.
// Square heads of 64 and 128 take a compile-time-shaped kernel (128: 512
// threads, 8 rows each), the rest a general one bounded by runtime sizes.
// q, k, v may be bf16, fp32 or FP8 (E4M3); they are decoded to fp32 exactly.
#include "lla_device.h"
#include "lla_internal.h"

namespace lla {

// GATED: S = g S + k v^T with one gate per (b,h) (see the gated prefill in
// lla_prefill.hip), g = gate[bh] taken in [2^-126, 1] like there.
template <typename Tin, int VW, int RPT, bool GATED = false>
__global__ __launch_bounds__(kThreads) void k_decode_step(const Tin* __restrict__ q,
                                                          const Tin* __restrict__ k,
                                                          const Tin* __restrict__ v,
                                                          float* __restrict__ S,
                                                          float* __restrict__ o, int dk, int dv,
                                                          const float* __restrict__ gate) {
    typedef float vecf __attribute__((ext_vector_type(VW)));
    __shared__ float qs[128], ks[128], vs[128];
    __shared__ float red[kThreads * VW];

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    for (int i = tid; i < dk; i += kThreads) {
        qs[i] = to_f32(q[bh * dk + i]);
        ks[i] = to_f32(k[bh * dk + i]);
    }
    for (int j = tid; j < dv; j += kThreads) vs[j] = to_f32(v[bh * dv + j]);
    __syncthreads();

    const int ncg = (dv + VW - 1) / VW;  // column groups
    const int rg_n = kThreads / ncg;     // row groups
    const int cg = tid % ncg, rg = tid / ncg;
    const bool active = rg < rg_n;
    const int j0 = cg * VW;
    float* Sb = S + bh * (int64_t)dk * dv;
    float gm = 1.0f;
    if constexpr (GATED) gm = decay_gate(gate[bh]);

    vecf vj;
#pragma unroll
    for (int u = 0; u < VW; ++u) vj[u] = (j0 + u < dv) ? vs[j0 + u] : 0.0f;
    vecf acc = {};

    if (active) {
        for (int i0 = rg; i0 < dk; i0 += rg_n * RPT) {
            vecf s[RPT];
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int i = i0 + m * rg_n;
                if (i < dk) {
                    if constexpr (VW == 4)
                        s[m] = __builtin_nontemporal_load(reinterpret_cast<const vecf*>(Sb + (int64_t)i * dv + j0));
                    else
                        s[m] = Sb[(int64_t)i * dv + j0];
                }
            }
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int i = i0 + m * rg_n;
                if (i < dk) {
                    const float ki = ks[i], qi = qs[i];
#pragma unroll
                    for (int u = 0; u < VW; ++u) {
                        if constexpr (GATED) s[m][u] = gm * s[m][u];  // decay
                        s[m][u] = fmaf(ki, vj[u], s[m][u]);  // rank-1 update
                        acc[u] = fmaf(qi, s[m][u], acc[u]);  // state read
                    }
                    if constexpr (VW == 4)
                        __builtin_nontemporal_store(s[m], reinterpret_cast<vecf*>(Sb + (int64_t)i * dv + j0));
                    else
                        Sb[(int64_t)i * dv + j0] = s[m][0];
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < VW; ++u) red[tid * VW + u] = active ? acc[u] : 0.0f;
    __syncthreads();
    // o[j] = sum over row groups, in row-group order
    for (int j = tid; j < dv; j += kThreads) {
        const int c = j / VW, u = j % VW;
        float sum = 0.0f;
        for (int r = 0; r < rg_n; ++r) sum += red[(r * ncg + c) * VW + u];
        o[bh * dv + j] = sum;
    }
}

// Compile-time shape for the common case dk = dv = D (D a multiple of 4):
// NT threads = (D/4) column groups x RG row groups, RPT = D/RG rows each.
// All RPT 16-byte state loads of a thread are issued before the first use.
template <typename Tin, int D, int NT, bool GATED = false>
__global__ __launch_bounds__(NT) void k_decode_step_sq(const Tin* __restrict__ q,
                                                      const Tin* __restrict__ k,
                                                      const Tin* __restrict__ v,
                                                      float* __restrict__ S,
                                                      float* __restrict__ o,
                                                      const float* __restrict__ gate) {
    constexpr int CG = D / 4, RG = NT / CG, RPT = D / RG;
    static_assert(NT % CG == 0 && D % RG == 0, "thread layout must tile the state");
    __shared__ float qs[D], ks[D], vs[D];
    __shared__ f32x4 red[RG][CG];
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    const int64_t bh = blockIdx.x;
    float* Sb = S + bh * (int64_t)D * D;
    // q, k, v go to LDS first and the state stream starts after the barrier,
    // so that the waves of a workgroup issue it together: issuing the state
    // loads ahead of the barrier measured about 8% slower.
    for (int i = tid; i < D; i += NT) {
        qs[i] = to_f32(q[bh * D + i]);
        ks[i] = to_f32(k[bh * D + i]);
        vs[i] = to_f32(v[bh * D + i]);
    }
    __syncthreads();
    f32x4 x[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        x[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (rg + m * RG) * D + 4 * cg));
    const f32x4 vj = {vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3]};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float gm = 1.0f;
    if constexpr (GATED) gm = decay_gate(gate[bh]);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const float ki = ks[i], qi = qs[i];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if constexpr (GATED) x[m][u] = gm * x[m][u];  // decay
            x[m][u] = fmaf(ki, vj[u], x[m][u]);  // rank-1 update
            acc[u] = fmaf(qi, x[m][u], acc[u]);  // state read
        }
        __builtin_nontemporal_store(x[m], reinterpret_cast<f32x4*>(Sb + i * D + 4 * cg));
    }
    red[rg][cg] = acc;
    __syncthreads();
    for (int j = tid; j < D; j += NT) {  // o[j] = sum over row groups, in order
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < RG; ++r) sum += red[r][j / 4][j % 4];
        o[bh * D + j] = sum;
    }
}


// Several tokens per call (a short continuation from an existing state:
// deck "Mechanism map", decode line, applied T times).  The state slice stays
// in registers across the T steps -- one state read and one write for all T
// tokens.  Each step is the decode step above with the same per-element
// arithmetic and the same reduction order, so T = 1 gives identical bits.
// With shared-state heads (G query heads per key/value head, as in
// k_decode_group below) every step updates the state once and then reads it
// for each of the G query heads, as k_decode_group does.
// One workgroup per key/value head bh: k, v rows bh * T + t; q, o rows
// (bh * G + g) * T + t (the query heads of a group are consecutive);
// T <= TMAX.  The query heads of a step are reduced GB at a time (one LDS
// reduction, two barriers, per batch).  Query rows: with GQ = 0 all T * G
// (<= QMAX) are staged up front; with GQ > 0 (G <= GQ) only the G rows of the
// current and of the next token are staged, double-buffered, and the next
// token's rows are fetched while the current token updates the state -- the
// smaller LDS footprint lets more workgroups share a CU.
template <typename Tin, int D, int NT, int TMAX, int QMAX, int GB, int GQ>
__global__ __launch_bounds__(NT) void k_decode_tokens(const Tin* __restrict__ q,
                                                      const Tin* __restrict__ k,
                                                      const Tin* __restrict__ v,
                                                      float* __restrict__ S,
                                                      float* __restrict__ o, int T, int G,
                                                      int mode) {
    // mode bit 0: S_0 = 0 (S is not read); bit 1: S is not written (a verify
    // pass over draft tokens, lla_prefill_ex with LLA_PREFILL_KEEP_STATE)
    const bool zero_start = (mode & 1) != 0, keep_state = (mode & 2) != 0;
    constexpr int CG = D / 4, RG = NT / CG, RPT = D / RG;
    static_assert(NT % CG == 0 && D % RG == 0, "thread layout must tile the state");
    constexpr int QROWS = GQ > 0 ? 2 * GQ : QMAX;             // staged query rows
    constexpr int QPT = GQ > 0 ? (GQ * D + NT - 1) / NT : 1;  // next-token q elements per thread
    // qs row t * G + g (GQ = 0), or (t & 1) * GQ + g (GQ > 0)
    __shared__ float qs[QROWS][D], ks[TMAX][D], vs[TMAX][D];
    __shared__ f32x4 red[GB][RG][CG];
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    const int64_t bh = blockIdx.x;
    float* Sb = S + bh * (int64_t)D * D;
    const int64_t tok0 = bh * T;  // first k, v row of this key/value head
    for (int e = tid; e < T * D; e += NT) {
        const int t = e / D, i = e % D;
        ks[t][i] = to_f32(k[tok0 * D + e]);
        vs[t][i] = to_f32(v[tok0 * D + e]);
    }
    if constexpr (GQ == 0) {
        for (int e = tid; e < G * T * D; e += NT) {
            const int g = e / (T * D), r = e % (T * D), t = r / D, i = r % D;
            qs[t * G + g][i] = to_f32(q[(bh * G + g) * (int64_t)T * D + r]);
        }
    } else {  // token 0's rows into buffer 0
        for (int e = tid; e < G * D; e += NT)
            qs[e / D][e % D] = to_f32(q[(bh * G + e / D) * (int64_t)T * D + e % D]);
    }
    __syncthreads();
    f32x4 x[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        x[m] = zero_start ? f32x4{0.f, 0.f, 0.f, 0.f}  // S_0 = 0: S is not read
                          : __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (rg + m * RG) * D + 4 * cg));
    for (int t = 0; t < T; ++t) {
        float qn[QPT];  // the next token's query rows, on their way to LDS
        if constexpr (GQ > 0) {
            if (t + 1 < T) {
#pragma unroll
                for (int n = 0; n < QPT; ++n) {
                    const int e = tid + n * NT;
                    if (e < G * D) qn[n] = to_f32(q[((bh * G + e / D) * (int64_t)T + t + 1) * D + e % D]);
                }
            }
        }
        const f32x4 vj = {vs[t][4 * cg], vs[t][4 * cg + 1], vs[t][4 * cg + 2], vs[t][4 * cg + 3]};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float ki = ks[t][rg + m * RG];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[m][u] = fmaf(ki, vj[u], x[m][u]);  // rank-1 update
        }
        if constexpr (GQ > 0) {
            // buffer (t + 1) & 1 was last read by token t - 1, before the
            // barriers that ended it; the barriers below publish it
            if (t + 1 < T) {
#pragma unroll
                for (int n = 0; n < QPT; ++n) {
                    const int e = tid + n * NT;
                    if (e < G * D) qs[((t + 1) & 1) * GQ + e / D][e % D] = qn[n];
                }
            }
        }
        const int qrow0 = GQ > 0 ? (t & 1) * GQ : t * G;
        for (int g0 = 0; g0 < G; g0 += GB) {
            const int nb = min(GB, G - g0);
#pragma unroll
            for (int b = 0; b < GB; ++b) {
                if (b >= nb) break;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const float qi = qs[qrow0 + g0 + b][rg + m * RG];
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[u] = fmaf(qi, x[m][u], acc[u]);  // state read
                }
                red[b][rg][cg] = acc;
            }
            __syncthreads();
            for (int e = tid; e < nb * D; e += NT) {  // o_t[j] = sum over row groups, in order
                const int b = e / D, j = e % D;
                float sum = 0.0f;
#pragma unroll
                for (int r = 0; r < RG; ++r) sum += red[b][r][j / 4][j % 4];
                o[((bh * G + g0 + b) * T + t) * (int64_t)D + j] = sum;
            }
            __syncthreads();  // red is rewritten by the next batch or token
        }
    }
    if (keep_state) return;
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_nontemporal_store(x[m], reinterpret_cast<f32x4*>(Sb + (rg + m * RG) * D + 4 * cg));
}


// Shared-state heads (query heads grouped on one key/value head, as in
// grouped-query attention): the state is updated once and then read by each
// of the group's G query heads.  Query head g of state bh is row bh * G + g
// of q and o.  For every query head the arithmetic (update, then the state
// read in row order, then the row-group reduction) is that of
// k_decode_step_sq, so a group of one gives identical bits.  The query rows
// are staged in LDS GMAX at a time.  GATED: S = g S + k v^T with one gate per
// key/value head (gate[bh]), as in the gated step.
template <typename Tin, int D, int NT, int GMAX, bool GATED = false>
__global__ __launch_bounds__(NT) void k_decode_group(const Tin* __restrict__ q,
                                                     const Tin* __restrict__ k,
                                                     const Tin* __restrict__ v,
                                                     float* __restrict__ S,
                                                     float* __restrict__ o, int G,
                                                     const float* __restrict__ gate) {
    constexpr int CG = D / 4, RG = NT / CG, RPT = D / RG;
    static_assert(NT % CG == 0 && D % RG == 0, "thread layout must tile the state");
    __shared__ float qs[GMAX][D], ks[D], vs[D];
    __shared__ f32x4 red[RG][CG];
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    const int64_t bh = blockIdx.x;
    float* Sb = S + bh * (int64_t)D * D;
    const int nb0 = G < GMAX ? G : GMAX;
    for (int e = tid; e < nb0 * D; e += NT) qs[e / D][e % D] = to_f32(q[bh * G * D + e]);
    for (int i = tid; i < D; i += NT) {
        ks[i] = to_f32(k[bh * D + i]);
        vs[i] = to_f32(v[bh * D + i]);
    }
    __syncthreads();
    f32x4 x[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        x[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (rg + m * RG) * D + 4 * cg));
    const f32x4 vj = {vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3]};
    float gm = 1.0f;
    if constexpr (GATED) gm = decay_gate(gate[bh]);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const float ki = ks[i];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if constexpr (GATED) x[m][u] = gm * x[m][u];  // decay
            x[m][u] = fmaf(ki, vj[u], x[m][u]);          // rank-1 update
        }
        __builtin_nontemporal_store(x[m], reinterpret_cast<f32x4*>(Sb + i * D + 4 * cg));
    }
    for (int g0 = 0; g0 < G; g0 += GMAX) {
        const int nb = G - g0 < GMAX ? G - g0 : GMAX;
        if (g0 > 0) {  // the previous batch's last barrier ended every read of qs
            for (int e = tid; e < nb * D; e += NT) qs[e / D][e % D] = to_f32(q[(bh * G + g0) * D + e]);
            __syncthreads();
        }
        for (int g = 0; g < nb; ++g) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const float qi = qs[g][rg + m * RG];
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[u] = fmaf(qi, x[m][u], acc[u]);  // state read
            }
            red[rg][cg] = acc;
            __syncthreads();
            for (int j = tid; j < D; j += NT) {  // o[j] = sum over row groups, in order
                float sum = 0.0f;
#pragma unroll
                for (int r = 0; r < RG; ++r) sum += red[r][j / 4][j % 4];
                o[(bh * G + g0 + g) * D + j] = sum;
            }
            __syncthreads();  // red (and, after the last head, qs) is rewritten next
        }
    }
}

// Shared-state heads for the other head dims (dk, dv <= 128): the thread
// layout and arithmetic of k_decode_step (VW value columns per thread,
// row groups of rg_n, rows rg + m * rg_n), with all of a thread's rows in
// registers at once (RPT * rg_n >= dk, checked by the launcher), so every
// query head's o has the bits of a plain decode step on the updated state.
// The query rows are staged in LDS GB at a time.  GATED as k_decode_group.
template <typename Tin, int VW, int RPT, int GB, bool GATED = false>
__global__ __launch_bounds__(kThreads) void k_decode_group_any(const Tin* __restrict__ q,
                                                               const Tin* __restrict__ k,
                                                               const Tin* __restrict__ v,
                                                               float* __restrict__ S,
                                                               float* __restrict__ o, int dk, int dv, int G,
                                                               const float* __restrict__ gate) {
    typedef float vecf __attribute__((ext_vector_type(VW)));
    __shared__ float qs[GB][128], ks[128], vs[128];
    __shared__ float red[kThreads * VW];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    for (int i = tid; i < dk; i += kThreads) ks[i] = to_f32(k[bh * dk + i]);
    for (int j = tid; j < dv; j += kThreads) vs[j] = to_f32(v[bh * dv + j]);
    __syncthreads();
    const int ncg = (dv + VW - 1) / VW;  // column groups
    const int rg_n = kThreads / ncg;     // row groups
    const int cg = tid % ncg, rg = tid / ncg;
    const bool active = rg < rg_n;
    const int j0 = cg * VW;
    float* Sb = S + bh * (int64_t)dk * dv;
    vecf vj;
#pragma unroll
    for (int u = 0; u < VW; ++u) vj[u] = (j0 + u < dv) ? vs[j0 + u] : 0.0f;
    vecf s[RPT];
    if (active) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + m * rg_n;
            if (i < dk) {
                if constexpr (VW == 4)
                    s[m] = __builtin_nontemporal_load(reinterpret_cast<const vecf*>(Sb + (int64_t)i * dv + j0));
                else
                    s[m] = Sb[(int64_t)i * dv + j0];
            }
        }
        float gm = 1.0f;
        if constexpr (GATED) gm = decay_gate(gate[bh]);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + m * rg_n;
            if (i < dk) {
                const float ki = ks[i];
#pragma unroll
                for (int u = 0; u < VW; ++u) {
                    if constexpr (GATED) s[m][u] = gm * s[m][u];  // decay
                    s[m][u] = fmaf(ki, vj[u], s[m][u]);          // rank-1 update
                }
                if constexpr (VW == 4)
                    __builtin_nontemporal_store(s[m], reinterpret_cast<vecf*>(Sb + (int64_t)i * dv + j0));
                else
                    Sb[(int64_t)i * dv + j0] = s[m][0];
            }
        }
    }
    for (int g0 = 0; g0 < G; g0 += GB) {
        const int nb = G - g0 < GB ? G - g0 : GB;
        for (int e = tid; e < nb * dk; e += kThreads) qs[e / dk][e % dk] = to_f32(q[(bh * G + g0) * dk + e]);
        __syncthreads();  // the previous batch's last barrier ended every read of qs
        for (int g = 0; g < nb; ++g) {
            vecf acc = {};
            if (active) {
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const int i = rg + m * rg_n;
                    if (i < dk) {
                        const float qi = qs[g][i];
#pragma unroll
                        for (int u = 0; u < VW; ++u) acc[u] = fmaf(qi, s[m][u], acc[u]);  // state read
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < VW; ++u) red[tid * VW + u] = acc[u];
            __syncthreads();
            for (int j = tid; j < dv; j += kThreads) {  // o[j] = sum over row groups, in order
                const int c = j / VW, u = j % VW;
                float sum = 0.0f;
                for (int r = 0; r < rg_n; ++r) sum += red[(r * ncg + c) * VW + u];
                o[(bh * G + g0 + g) * dv + j] = sum;
            }
            __syncthreads();  // red (and, after the last head, qs) is rewritten next
        }
    }
}

// The commit after a verify pass over T draft tokens (speculative decoding):
// S += sum over the first m accepted tokens t of k_t v_t^T, per state element
// in token order with one fmaf each -- exactly the update of m decode steps
// (lla_decode_step), so the state after the commit equals the state after m
// decode steps bit for bit.  m = accepted[sequence], clamped to [0, T], or T
// when accepted is null; m = 0 leaves the state unread and unwritten.
// One workgroup per key/value head bh (sequence bh / Hkv); k, v rows
// bh * T + t.  A thread owns VEC consecutive elements of a row (VEC = 4 when
// dv is a multiple of 4, else 1) at a stride of kThreads * VEC elements.
// GATED: the gated commit, S <- g_t S + k_t v_t^T per accepted token with
// g_t = gate[bh * T + t] (taken in [2^-126, 1]), the arithmetic of the gated
// decode step, so the state equals m gated decode steps' bit for bit.
template <typename Tin, int VEC, bool GATED = false>
__global__ __launch_bounds__(kThreads) void k_state_commit(const Tin* __restrict__ k,
                                                          const Tin* __restrict__ v,
                                                          const int32_t* __restrict__ accepted,
                                                          float* __restrict__ S, int T, int Hkv,
                                                          int dk, int dv, const float* __restrict__ gate) {
    constexpr int TB = 16;          // tokens staged per pass
    constexpr int NE = 128 * 128 / (kThreads * VEC);  // element groups per thread at most
    __shared__ float ks[TB][128], vs[TB][128], gs[TB];
    typedef float vecf __attribute__((ext_vector_type(VEC)));
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    int m = accepted ? accepted[bh / Hkv] : T;
    m = m < 0 ? 0 : (m > T ? T : m);
    if (m == 0) return;  // uniform over the workgroup
    float* Sb = S + bh * (int64_t)dk * dv;
    const int ngrp = dk * dv / VEC;  // VEC divides dv, so a group stays in one row
    vecf x[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int e = tid + n * kThreads;
        if (e < ngrp) x[n] = *reinterpret_cast<const vecf*>(Sb + (int64_t)e * VEC);
    }
    for (int t0 = 0; t0 < m; t0 += TB) {
        const int nt = m - t0 < TB ? m - t0 : TB;
        __syncthreads();  // the previous pass is done with ks, vs
        for (int e = tid; e < nt * dk; e += kThreads)
            ks[e / dk][e % dk] = to_f32(k[(bh * T + t0 + e / dk) * (int64_t)dk + e % dk]);
        for (int e = tid; e < nt * dv; e += kThreads)
            vs[e / dv][e % dv] = to_f32(v[(bh * T + t0 + e / dv) * (int64_t)dv + e % dv]);
        if constexpr (GATED)
            if (tid < nt) gs[tid] = decay_gate(gate[bh * T + t0 + tid]);
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            float gm = 1.0f;
            if constexpr (GATED) gm = gs[t];
#pragma unroll
            for (int n = 0; n < NE; ++n) {
                const int e = tid + n * kThreads;
                if (e < ngrp) {
                    const int i = e * VEC / dv, j = e * VEC % dv;
                    const float ki = ks[t][i];
#pragma unroll
                    for (int u = 0; u < VEC; ++u) {
                        if constexpr (GATED) x[n][u] = gm * x[n][u];  // decay
                        x[n][u] = fmaf(ki, vs[t][j + u], x[n][u]);    // rank-1 update
                    }
                }
            }
        }
    }
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int e = tid + n * kThreads;
        if (e < ngrp) *reinterpret_cast<vecf*>(Sb + (int64_t)e * VEC) = x[n];
    }
}

// The same commit for square heads of 64 and 128 in the decode step's
// layout (k_decode_step_sq): NT threads = (D/4) column groups x RG row
// groups, each thread RPT rows of one 16-byte column group, all of its state
// loads issued before the first use, streaming loads and stores.  Per
// element the arithmetic is that of k_state_commit (one fmaf per token in
// token order), so the two give identical bits (GATED: with the decay
// first, as there).
template <typename Tin, int D, int NT, bool GATED = false>
__global__ __launch_bounds__(NT) void k_state_commit_sq(const Tin* __restrict__ k,
                                                       const Tin* __restrict__ v,
                                                       const int32_t* __restrict__ accepted,
                                                       float* __restrict__ S, int T, int Hkv,
                                                       const float* __restrict__ gate) {
    constexpr int CG = D / 4, RG = NT / CG, RPT = D / RG;
    static_assert(NT % CG == 0 && D % RG == 0, "thread layout must tile the state");
    constexpr int TB = 16;  // tokens staged per pass
    __shared__ float ks[TB][D], vs[TB][D], gs[TB];
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    const int64_t bh = blockIdx.x;
    int m = accepted ? accepted[bh / Hkv] : T;
    m = m < 0 ? 0 : (m > T ? T : m);
    if (m == 0) return;  // uniform over the workgroup
    float* Sb = S + bh * (int64_t)D * D;
    f32x4 x[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        x[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (rg + r * RG) * D + 4 * cg));
    for (int t0 = 0; t0 < m; t0 += TB) {
        const int nt = m - t0 < TB ? m - t0 : TB;
        __syncthreads();  // the previous pass is done with ks, vs
        for (int e = tid; e < nt * D; e += NT) {
            ks[e / D][e % D] = to_f32(k[(bh * T + t0) * D + e]);
            vs[e / D][e % D] = to_f32(v[(bh * T + t0) * D + e]);
        }
        if constexpr (GATED)
            if (tid < nt) gs[tid] = decay_gate(gate[bh * T + t0 + tid]);
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            const f32x4 vj = {vs[t][4 * cg], vs[t][4 * cg + 1], vs[t][4 * cg + 2], vs[t][4 * cg + 3]};
            float gm = 1.0f;
            if constexpr (GATED) gm = gs[t];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const float ki = ks[t][rg + r * RG];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if constexpr (GATED) x[r][u] = gm * x[r][u];  // decay
                    x[r][u] = fmaf(ki, vj[u], x[r][u]);          // rank-1 update
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        __builtin_nontemporal_store(x[r], reinterpret_cast<f32x4*>(Sb + (rg + r * RG) * D + 4 * cg));
}

template <typename Tin, bool GATED>
static hipError_t commit_t(const void* k, const void* v, const int32_t* accepted, int64_t BHkv, int Hkv,
                           int T, int dk, int dv, float* S, const float* gate, hipStream_t st) {
    if (dk == 128 && dv == 128)
        hipLaunchKernelGGL((k_state_commit_sq<Tin, 128, 512, GATED>), dim3((unsigned)BHkv), dim3(512), 0, st,
                           (const Tin*)k, (const Tin*)v, accepted, S, T, Hkv, gate);
    else if (dk == 64 && dv == 64)
        hipLaunchKernelGGL((k_state_commit_sq<Tin, 64, 256, GATED>), dim3((unsigned)BHkv), dim3(256), 0, st,
                           (const Tin*)k, (const Tin*)v, accepted, S, T, Hkv, gate);
    else if ((dv & 3) == 0)
        hipLaunchKernelGGL((k_state_commit<Tin, 4, GATED>), dim3((unsigned)BHkv), dim3(kThreads), 0, st,
                           (const Tin*)k, (const Tin*)v, accepted, S, T, Hkv, dk, dv, gate);
    else
        hipLaunchKernelGGL((k_state_commit<Tin, 1, GATED>), dim3((unsigned)BHkv), dim3(kThreads), 0, st,
                           (const Tin*)k, (const Tin*)v, accepted, S, T, Hkv, dk, dv, gate);
    return hipGetLastError();
}

template <bool GATED>
static hipError_t commit_dt(lla_dtype dtype, const void* k, const void* v, const int32_t* accepted,
                            int64_t BHkv, int Hkv, int T, int dk, int dv, float* S, const float* gate,
                            hipStream_t st) {
    if (dtype == LLA_FP8_E4M3) return commit_t<fp8e4m3, GATED>(k, v, accepted, BHkv, Hkv, T, dk, dv, S, gate, st);
    if (dtype == LLA_BF16) return commit_t<bf16, GATED>(k, v, accepted, BHkv, Hkv, T, dk, dv, S, gate, st);
    return commit_t<float, GATED>(k, v, accepted, BHkv, Hkv, T, dk, dv, S, gate, st);
}

hipError_t launch_state_commit(lla_dtype dtype, const void* k, const void* v, const int32_t* accepted,
                               int64_t BHkv, int Hkv, int T, int dk, int dv, float* S, hipStream_t st) {
    return commit_dt<false>(dtype, k, v, accepted, BHkv, Hkv, T, dk, dv, S, nullptr, st);
}

hipError_t launch_state_commit_gated(lla_dtype dtype, const void* k, const void* v, const float* gate,
                                     const int32_t* accepted, int64_t BH, int H, int T, int dk, int dv,
                                     float* S, hipStream_t st) {
    return commit_dt<true>(dtype, k, v, accepted, BH, H, T, dk, dv, S, gate, st);
}

__global__ __launch_bounds__(kThreads) void k_fill_zero(float* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if ((n & 3) == 0) {
        f32x4* p4 = reinterpret_cast<f32x4*>(p);
        for (; i < n / 4; i += stride) p4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        for (; i < n; i += stride) p[i] = 0.0f;
    }
}

template <typename Tin, bool GATED>
static hipError_t decode_t(const void* q, const void* k, const void* v, int64_t BH, int dk,
                           int dv, float* S, float* o, const float* gate, hipStream_t st) {
    if (dk == 128 && dv == 128) {
        hipLaunchKernelGGL((k_decode_step_sq<Tin, 128, 512, GATED>), dim3((unsigned)BH), dim3(512), 0, st,
                           (const Tin*)q, (const Tin*)k, (const Tin*)v, S, o, gate);
    } else if (dk == 64 && dv == 64) {
        hipLaunchKernelGGL((k_decode_step_sq<Tin, 64, 256, GATED>), dim3((unsigned)BH), dim3(256), 0, st,
                           (const Tin*)q, (const Tin*)k, (const Tin*)v, S, o, gate);
    } else if ((dv & 3) == 0) {
        // 256 threads = (dv/4) column groups x rg row groups; RPT rows each
        // cover dk <= 128 in one batch when dv = 128 (8 row groups x 16).
        hipLaunchKernelGGL((k_decode_step<Tin, 4, 16, GATED>), dim3((unsigned)BH), dim3(kThreads), 0, st,
                           (const Tin*)q, (const Tin*)k, (const Tin*)v, S, o, dk, dv, gate);
    } else {
        hipLaunchKernelGGL((k_decode_step<Tin, 1, 4, GATED>), dim3((unsigned)BH), dim3(kThreads), 0, st,
                           (const Tin*)q, (const Tin*)k, (const Tin*)v, S, o, dk, dv, gate);
    }
    return hipGetLastError();
}

hipError_t launch_decode_step(lla_dtype dtype, const void* q, const void* k, const void* v,
                              int64_t BH, int dk, int dv, float* S, float* o, hipStream_t st) {
    if (dtype == LLA_FP8_E4M3) return decode_t<fp8e4m3, false>(q, k, v, BH, dk, dv, S, o, nullptr, st);
    if (dtype == LLA_BF16) return decode_t<bf16, false>(q, k, v, BH, dk, dv, S, o, nullptr, st);
    return decode_t<float, false>(q, k, v, BH, dk, dv, S, o, nullptr, st);
}

hipError_t launch_decode_step_gated(lla_dtype dtype, const void* q, const void* k, const void* v,
                                    const float* gate, int64_t BH, int dk, int dv, float* S, float* o,
                                    hipStream_t st) {
    if (dtype == LLA_FP8_E4M3) return decode_t<fp8e4m3, true>(q, k, v, BH, dk, dv, S, o, gate, st);
    if (dtype == LLA_BF16) return decode_t<bf16, true>(q, k, v, BH, dk, dv, S, o, gate, st);
    return decode_t<float, true>(q, k, v, BH, dk, dv, S, o, gate, st);
}

bool decode_tokens_fit(int64_t T, int dk, int dv, int64_t group) {
    return T >= 1 && T <= kDecodeTokensMax && group >= 1 && group <= kDecodeGroupMax &&
           T * group <= kDecodeTokensQueries && dk == dv && (dk == 64 || dk == 128);
}

template <typename Tin, int QMAX, int GB, int GQ>
static hipError_t tokens_t(const void* q, const void* k, const void* v, int64_t BHkv, int T, int G,
                           int d, float* S, float* o, int zero, hipStream_t st) {
    if (d == 128)
        hipLaunchKernelGGL((k_decode_tokens<Tin, 128, 512, kDecodeTokensMax, QMAX, GB, GQ>), dim3((unsigned)BHkv),
                           dim3(512), 0, st, (const Tin*)q, (const Tin*)k, (const Tin*)v, S, o, T, G, zero);
    else
        hipLaunchKernelGGL((k_decode_tokens<Tin, 64, 256, kDecodeTokensMax, QMAX, GB, GQ>), dim3((unsigned)BHkv),
                           dim3(256), 0, st, (const Tin*)q, (const Tin*)k, (const Tin*)v, S, o, T, G, zero);
    return hipGetLastError();
}

template <typename Tin>
static hipError_t tokens_g(const void* q, const void* k, const void* v, int64_t BHkv, int T, int G,
                           int d, float* S, float* o, int zero, hipStream_t st) {
    // One query head per state: all query rows are staged up front, no more
    // than the k, v rows.  Groups stage the query rows of two tokens at a
    // time; up to four heads per state reduce two heads per LDS pass (37 KB
    // of LDS at d = 128: four workgroups per CU), larger groups four.
    if (G == 1) return tokens_t<Tin, kDecodeTokensMax, 1, 0>(q, k, v, BHkv, T, G, d, S, o, zero, st);
    if (G <= 4) return tokens_t<Tin, kDecodeTokensQueries, 2, 4>(q, k, v, BHkv, T, G, d, S, o, zero, st);
    return tokens_t<Tin, kDecodeTokensQueries, 4, kDecodeGroupMax>(q, k, v, BHkv, T, G, d, S, o, zero, st);
}

hipError_t launch_decode_tokens(lla_dtype dtype, const void* q, const void* k, const void* v,
                                int64_t BHkv, int T, int group, int d, float* S, float* o,
                                bool zero_start, bool keep_state, hipStream_t st) {
    const int z = (zero_start ? 1 : 0) | (keep_state ? 2 : 0);
    if (dtype == LLA_FP8_E4M3) return tokens_g<fp8e4m3>(q, k, v, BHkv, T, group, d, S, o, z, st);
    if (dtype == LLA_BF16) return tokens_g<bf16>(q, k, v, BHkv, T, group, d, S, o, z, st);
    return tokens_g<float>(q, k, v, BHkv, T, group, d, S, o, z, st);
}

// Rows per thread that k_decode_group_any needs to hold a whole dk x dv
// state in one pass with VW columns per thread.
static int group_any_rows(int dk, int dv, int VW) {
    const int ncg = (dv + VW - 1) / VW, rg_n = kThreads / ncg;
    return (dk + rg_n - 1) / rg_n;
}

template <typename Tin, bool GATED>
static hipError_t group_t(const void* q, const void* k, const void* v, int64_t BHkv, int G, int dk, int dv,
                          float* S, float* o, const float* gate, hipStream_t st) {
    const Tin *qq = (const Tin*)q, *kk = (const Tin*)k, *vv = (const Tin*)v;
    const dim3 grid((unsigned)BHkv);
    if (dk == 128 && dv == 128)
        hipLaunchKernelGGL((k_decode_group<Tin, 128, 512, kDecodeGroupBatch, GATED>), grid, dim3(512), 0, st, qq, kk,
                           vv, S, o, G, gate);
    else if (dk == 64 && dv == 64)
        hipLaunchKernelGGL((k_decode_group<Tin, 64, 256, kDecodeGroupBatch, GATED>), grid, dim3(256), 0, st, qq, kk,
                           vv, S, o, G, gate);
    else if ((dv & 3) == 0) {
        // dv / 4 <= 32 column groups leave >= 8 row groups: 16 rows each cover dk <= 128
        if (group_any_rows(dk, dv, 4) > 16) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_decode_group_any<Tin, 4, 16, kDecodeGroupBatch, GATED>), grid, dim3(kThreads), 0, st,
                           qq, kk, vv, S, o, dk, dv, G, gate);
    } else {
        // dv <= 128 columns leave >= 2 row groups: 64 rows each cover dk <= 128
        if (group_any_rows(dk, dv, 1) > 64) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_decode_group_any<Tin, 1, 64, kDecodeGroupBatch, GATED>), grid, dim3(kThreads), 0, st,
                           qq, kk, vv, S, o, dk, dv, G, gate);
    }
    return hipGetLastError();
}

template <bool GATED>
static hipError_t group_dt(lla_dtype dtype, const void* q, const void* k, const void* v, int64_t BHkv, int group,
                           int dk, int dv, float* S, float* o, const float* gate, hipStream_t st) {
    if (dtype == LLA_FP8_E4M3) return group_t<fp8e4m3, GATED>(q, k, v, BHkv, group, dk, dv, S, o, gate, st);
    if (dtype == LLA_BF16) return group_t<bf16, GATED>(q, k, v, BHkv, group, dk, dv, S, o, gate, st);
    return group_t<float, GATED>(q, k, v, BHkv, group, dk, dv, S, o, gate, st);
}

hipError_t launch_decode_group(lla_dtype dtype, const void* q, const void* k, const void* v,
                               int64_t BHkv, int group, int dk, int dv, float* S, float* o, hipStream_t st) {
    return group_dt<false>(dtype, q, k, v, BHkv, group, dk, dv, S, o, nullptr, st);
}

hipError_t launch_decode_group_gated(lla_dtype dtype, const void* q, const void* k, const void* v,
                                     const float* gate, int64_t BHkv, int group, int dk, int dv, float* S,
                                     float* o, hipStream_t st) {
    return group_dt<true>(dtype, q, k, v, BHkv, group, dk, dv, S, o, gate, st);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t work = (n & 3) == 0 ? n / 4 : n;
    int64_t blocks = (work + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(kThreads), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace lla
