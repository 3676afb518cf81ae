// lla_prefill.hip -- chunkwise-parallel causal linear-attention prefill for
// gfx950 (MI355X).
//
// Method (slide deck "Chunking, causality, and parallel prefill"): per chunk c
// of C tokens, O_c = tril(Q_c K_c^T) V_c + Q_c S_c and S_{c+1} = S_c + K_c^T V_c
// ("Split into chunks", "Causal triangle", "Incoming and outgoing state");
// only the chunk-to-chunk state hop is serial.
//
// Three kernels:
//   k_segment_states : per (b,h) and segment of G chunks, the increment
//                      K_seg^T V_seg (fp32, matrix cores).
//   k_state_scan     : exclusive prefix over segments -> the state each
//                      segment starts from (the serial hop, one add per
//                      segment instead of one per chunk).
//   k_chunk_walk     : one workgroup per (b,h,segment) walks its G chunks with
//                      the fp32 state in registers: scores on matrix cores,
//                      causal mask in registers, masked scores times V plus
//                      Q times the state (state split into bf16 high + low
//                      parts), then the state hop K_c^T V_c.
//
// Matrix-core layout used throughout (16x16 tiles, 32-deep steps): see
// lla::mma.  The score tile is computed transposed (keys as rows), so that a
// lane ends up holding four consecutive key columns of one query row: those
// are stored to LDS as one 8-byte write, and the output tile is computed
// transposed as well (values as rows), so a lane holds four consecutive
// output columns: one 16-byte global store.
#include "lla_device.h"
#include "lla_internal.h"

#include <type_traits>

namespace lla {

template <typename T, int CT_, int D_>
struct WalkCfg {
    static constexpr int CT = CT_, D = D_;
    static constexpr bool BF = std::is_same<T, bf16>::value;
    static constexpr int LQ = D + (BF ? 8 : 4);   // Q/K LDS row stride: 16-byte rows
    static constexpr int LV = D + (BF ? 4 : 2);   // V LDS row stride: 8-byte rows, bank skew
    static constexpr int LP = CT + (BF ? 8 : 4);  // score LDS row stride
    static constexpr int NT = CT / 16;            // 16-row tiles per chunk
    static constexpr int NTS = CT / 32;           // 32-deep time steps per chunk
    static constexpr int NDT = D / 16;            // 16-wide tiles over the head dim
    static constexpr int NDS = D / 32;            // 32-deep steps over the head dim
    static constexpr int NVW = (NDT + kWaves - 1) / kWaves;  // value tiles per wave
    static constexpr int NTRI = NT * (NT + 1) / 2;           // lower-triangle tiles
    using Fr = typename Frag<T>::type;
};

// 8 consecutive elements from LDS (16-byte aligned) as one operand slice.
__device__ __forceinline__ bf16x8 lds_frag(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ f32x8 lds_frag(const float* p) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// 4 + 4 elements from two 8-byte aligned LDS addresses.
__device__ __forceinline__ bf16x8 lds_frag2(const bf16* p0, const bf16* p1) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 lds_frag2(const float* p0, const float* p1) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p1);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// 8 elements down a column (stride `ld` elements).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type lds_col(const T* p, int ld) {
    typename Frag<T>::type f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = p[s * ld];
    return f;
}
__device__ __forceinline__ void lds_store4(bf16* p, f32x4 x) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
}
__device__ __forceinline__ void lds_store4(float* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
}

// State hop for the tiles a wave owns: S[:, value tile w + 4*vw] += K^T V,
// contracting over the CT rows (time) of the staged tiles.
template <typename Cf, typename T>
__device__ __forceinline__ void state_hop(f32x4 (&Sacc)[Cf::NVW][Cf::NDT],
                                          const typename Cf::Fr (&Vf)[Cf::NVW][Cf::NTS],
                                          const T* Ks, int w, int g, int c16) {
#pragma unroll
    for (int dt = 0; dt < Cf::NDT; ++dt) {
#pragma unroll
        for (int ts = 0; ts < Cf::NTS; ++ts) {
            const typename Cf::Fr kt = lds_col(Ks + (32 * ts + 8 * g) * Cf::LQ + 16 * dt + c16, Cf::LQ);
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
                if (w + kWaves * vw < Cf::NDT) Sacc[vw][dt] = mma(kt, Vf[vw][ts], Sacc[vw][dt]);
        }
    }
}

// The value-column operand slices of a wave: V[32*ts + 8g + s][16*vt + c16].
template <typename Cf, typename T>
__device__ __forceinline__ void load_vfrags(typename Cf::Fr (&Vf)[Cf::NVW][Cf::NTS], const T* Vs,
                                            int w, int g, int c16) {
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) {
        const int vt = w + kWaves * vw;
#pragma unroll
        for (int ts = 0; ts < Cf::NTS; ++ts)
            if (vt < Cf::NDT) Vf[vw][ts] = lds_col(Vs + (32 * ts + 8 * g) * Cf::LV + 16 * vt + c16, Cf::LV);
    }
}

// ---------------------------------------------------------------------------
// Phase 1: per-segment state increments K_seg^T V_seg -> ws slot seg + 1.
// ---------------------------------------------------------------------------
template <typename T, int CT, int D>
__global__ __launch_bounds__(kThreads) void k_segment_states(
    const T* __restrict__ K, const T* __restrict__ V, float* __restrict__ ws, int64_t T_len,
    int dk, int dv, int C, int64_t G, int64_t n_seg, int vec) {
    using Cf = WalkCfg<T, CT, D>;
    using Fr = typename Cf::Fr;
    __shared__ __attribute__((aligned(16))) T Ks[CT * Cf::LQ];
    __shared__ __attribute__((aligned(16))) T Vs[CT * Cf::LV];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
    const int64_t nsm1 = n_seg - 1;
    const int64_t bh = blockIdx.x / nsm1, seg = blockIdx.x % nsm1;
    const int64_t n_c = (T_len + C - 1) / C;
    const int64_t c0 = seg * G, c1 = min(n_c, c0 + G);
    const T* Kb = K + bh * T_len * dk;
    const T* Vb = V + bh * T_len * dv;

    f32x4 Sacc[Cf::NVW][Cf::NDT];
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt) Sacc[vw][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    Tile<T, CT, D, Cf::LQ> tk;
    Tile<T, CT, D, Cf::LV> tv;
    auto rows_of = [&](int64_t c) { return (int)min((int64_t)C, T_len - c * C); };
    if (vec) {
        tk.gather(Kb + c0 * C * dk, dk, rows_of(c0), dk, tid);
        tv.gather(Vb + c0 * C * dv, dv, rows_of(c0), dv, tid);
    }
    for (int64_t c = c0; c < c1; ++c) {
        if (vec) {
            tk.scatter(Ks, tid);
            tv.scatter(Vs, tid);
        } else {
            Tile<T, CT, D, Cf::LQ>::load_scalar(Kb + c * C * dk, dk, rows_of(c), dk, Ks, tid);
            Tile<T, CT, D, Cf::LV>::load_scalar(Vb + c * C * dv, dv, rows_of(c), dv, Vs, tid);
        }
        __syncthreads();
        if (vec && c + 1 < c1) {
            tk.gather(Kb + (c + 1) * C * dk, dk, rows_of(c + 1), dk, tid);
            tv.gather(Vb + (c + 1) * C * dv, dv, rows_of(c + 1), dv, tid);
        }
        Fr Vf[Cf::NVW][Cf::NTS];
        load_vfrags<Cf>(Vf, Vs, w, g, c16);
        state_hop<Cf>(Sacc, Vf, Ks, w, g, c16);
        __syncthreads();
    }

    float* out = ws + (bh * n_seg + seg + 1) * (int64_t)dk * dv;
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) {
        const int v = 16 * (w + kWaves * vw) + c16;
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * dt + 4 * g + r;
                if (d < dk && v < dv) out[(int64_t)d * dv + v] = Sacc[vw][dt][r];
            }
    }
}

// ---------------------------------------------------------------------------
// Phase 2: slot 0 = S_0, slot s = S_0 + sum_{s' < s} increment(s').
// One thread per 4 consecutive state elements of one (b,h).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_state_scan(const float* __restrict__ S,
                                                         float* __restrict__ ws, int64_t n_seg,
                                                         int64_t dkdv, int64_t blocks_per_bh) {
    const int64_t bh = blockIdx.x / blocks_per_bh;
    const int64_t e = ((blockIdx.x % blocks_per_bh) * kThreads + threadIdx.x) * 4;
    if (e >= dkdv) return;
    float* slot = ws + bh * n_seg * dkdv + e;
    const float* s0 = S + bh * dkdv + e;
    if (e + 4 <= dkdv && (dkdv & 3) == 0) {
        f32x4 acc = *reinterpret_cast<const f32x4*>(s0);
        *reinterpret_cast<f32x4*>(slot) = acc;
        constexpr int U = 8;
        for (int64_t s = 1; s < n_seg; s += U) {
            f32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s + u < n_seg) x[u] = *reinterpret_cast<const f32x4*>(slot + (s + u) * dkdv);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s + u < n_seg) {
                    acc += x[u];
                    *reinterpret_cast<f32x4*>(slot + (s + u) * dkdv) = acc;
                }
        }
    } else {
        const int m = (int)min((int64_t)4, dkdv - e);
        for (int j = 0; j < m; ++j) {
            float acc = s0[j];
            slot[j] = acc;
            for (int64_t s = 1; s < n_seg; ++s) {
                acc += slot[s * dkdv + j];
                slot[s * dkdv + j] = acc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Phase 3: the chunk walk.  One workgroup per (b,h,segment); four waves; the
// fp32 state of the whole head lives in registers, split over the waves by
// value columns (wave w owns value tiles w, w+4, ...).
// ---------------------------------------------------------------------------
template <typename T, int CT, int D>
__global__ __launch_bounds__(kThreads) void k_chunk_walk(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    float* __restrict__ S, float* __restrict__ O, const float* __restrict__ ws, int64_t T_len,
    int dk, int dv, int C, int64_t G, int64_t n_seg, int vec) {
    using Cf = WalkCfg<T, CT, D>;
    using Fr = typename Cf::Fr;
    __shared__ __attribute__((aligned(16))) T Qs[CT * Cf::LQ];
    __shared__ __attribute__((aligned(16))) T Ks[CT * Cf::LQ];
    __shared__ __attribute__((aligned(16))) T Vs[CT * Cf::LV];
    __shared__ __attribute__((aligned(16))) T Ps[CT * Cf::LP];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
    const int64_t bh = blockIdx.x / n_seg, seg = blockIdx.x % n_seg;
    const int64_t n_c = (T_len + C - 1) / C;
    const int64_t c0 = seg * G, c1 = min(n_c, c0 + G);
    const bool last_seg = seg == n_seg - 1;
    const int64_t dkdv = (int64_t)dk * dv;
    const T* Qb = Q + bh * T_len * dk;
    const T* Kb = K + bh * T_len * dk;
    const T* Vb = V + bh * T_len * dv;
    float* Ob = O + bh * T_len * dv;

    // Incoming state of this segment.
    const float* Sin = n_seg == 1 ? S + bh * dkdv : ws + (bh * n_seg + seg) * dkdv;
    f32x4 Sacc[Cf::NVW][Cf::NDT];
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) {
        const int v = 16 * (w + kWaves * vw) + c16;
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * dt + 4 * g + r;
                Sacc[vw][dt][r] = (d < dk && v < dv) ? Sin[(int64_t)d * dv + v] : 0.0f;
            }
    }

    Tile<T, CT, D, Cf::LQ> tq, tk;
    Tile<T, CT, D, Cf::LV> tv;
    auto rows_of = [&](int64_t c) { return (int)min((int64_t)C, T_len - c * C); };
    if (vec) {
        tq.gather(Qb + c0 * C * dk, dk, rows_of(c0), dk, tid);
        tk.gather(Kb + c0 * C * dk, dk, rows_of(c0), dk, tid);
        tv.gather(Vb + c0 * C * dv, dv, rows_of(c0), dv, tid);
    }

    for (int64_t c = c0; c < c1; ++c) {
        const int nrows = rows_of(c);
        const int64_t t0 = c * C;
        if (vec) {
            tq.scatter(Qs, tid);
            tk.scatter(Ks, tid);
            tv.scatter(Vs, tid);
        } else {
            Tile<T, CT, D, Cf::LQ>::load_scalar(Qb + t0 * dk, dk, nrows, dk, Qs, tid);
            Tile<T, CT, D, Cf::LQ>::load_scalar(Kb + t0 * dk, dk, nrows, dk, Ks, tid);
            Tile<T, CT, D, Cf::LV>::load_scalar(Vb + t0 * dv, dv, nrows, dv, Vs, tid);
        }
        __syncthreads();
        if (vec && c + 1 < c1) {  // next chunk's loads fly during this chunk's math
            const int nr = rows_of(c + 1);
            tq.gather(Qb + (t0 + C) * dk, dk, nr, dk, tid);
            tk.gather(Kb + (t0 + C) * dk, dk, nr, dk, tid);
            tv.gather(Vb + (t0 + C) * dv, dv, nr, dv, tid);
        }

        // (1) Scores of the kept triangle, computed transposed: tile (jt, it)
        // holds A^T = K_c Q_c^T, i.e. lane (g, c16) has A[i][j] for query
        // i = 16 it + c16 and keys j = 16 jt + 4g + r.  Entries with j > i are
        // masked in registers; the rest is rounded to the input type (P).
        for (int e = w; e < Cf::NTRI; e += kWaves) {
            int it = 0;
            while ((it + 1) * (it + 2) / 2 <= e) ++it;
            const int jt = e - it * (it + 1) / 2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < Cf::NDS; ++ds)
                acc = mma(lds_frag(Ks + (16 * jt + c16) * Cf::LQ + 32 * ds + 8 * g),
                          lds_frag(Qs + (16 * it + c16) * Cf::LQ + 32 * ds + 8 * g), acc);
            const int i = 16 * it + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * jt + 4 * g + r > i) acc[r] = 0.0f;
            lds_store4(Ps + i * Cf::LP + 16 * jt + 4 * g, acc);
        }
        // Tiles right of the diagonal that a 32-deep step still reads: zero.
        for (int it = 2 * w; it + 1 < Cf::NT; it += 2 * kWaves)
            lds_store4(Ps + (16 * it + c16) * Cf::LP + 16 * (it + 1) + 4 * g, f32x4{0.f, 0.f, 0.f, 0.f});
        __syncthreads();

        // (2) Output, transposed: O^T tile (vt, it) = V^T P^T + S^T Q^T.
        Fr Vf[Cf::NVW][Cf::NTS];
        load_vfrags<Cf>(Vf, Vs, w, g, c16);

        // The state as the first operand: value row c16, depth slots
        // {4g + r} from tile 2ds and {16 + 4g + r} from tile 2ds + 1 -- exactly
        // the elements the lane already holds.  bf16 inputs: S = hi + lo.
        Fr Shi[Cf::NVW][Cf::NDS], Slo[Cf::NVW][Cf::NDS];
#pragma unroll
        for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
            for (int ds = 0; ds < Cf::NDS; ++ds)
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float x = Sacc[vw][2 * ds + (s >> 2)][s & 3];
                    if constexpr (Cf::BF) {
                        const bf16 h = to_bf16(x);
                        Shi[vw][ds][s] = h;
                        Slo[vw][ds][s] = to_bf16(x - to_f32(h));
                    } else {
                        Shi[vw][ds][s] = x;
                    }
                }

#pragma unroll
        for (int it = 0; it < Cf::NT; ++it) {
            f32x4 acc[Cf::NVW];
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw) acc[vw] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int i = 16 * it + c16;
            // masked scores times values: only time steps at or left of the diagonal
#pragma unroll
            for (int ts = 0; ts <= it / 2; ++ts) {
                const Fr pb = lds_frag(Ps + i * Cf::LP + 32 * ts + 8 * g);
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw)
                    if (w + kWaves * vw < Cf::NDT) acc[vw] = mma(Vf[vw][ts], pb, acc[vw]);
            }
            // incoming state read: Q_c S_c
#pragma unroll
            for (int ds = 0; ds < Cf::NDS; ++ds) {
                const Fr qb = lds_frag2(Qs + i * Cf::LQ + 32 * ds + 4 * g,
                                        Qs + i * Cf::LQ + 32 * ds + 16 + 4 * g);
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw)
                    if (w + kWaves * vw < Cf::NDT) {
                        acc[vw] = mma(Shi[vw][ds], qb, acc[vw]);
                        if constexpr (Cf::BF) acc[vw] = mma(Slo[vw][ds], qb, acc[vw]);
                    }
            }
            // lane holds O[t0 + i][16 vt + 4g + r], r = 0..3
            if (i < nrows) {
                float* orow = Ob + (t0 + i) * dv;
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw) {
                    const int v = 16 * (w + kWaves * vw) + 4 * g;
                    if (w + kWaves * vw < Cf::NDT && v < dv) {
                        if ((dv & 3) == 0) {
                            __builtin_nontemporal_store(acc[vw], reinterpret_cast<f32x4*>(orow + v));
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (v + r < dv) orow[v + r] = acc[vw][r];
                        }
                    }
                }
            }
        }

        // (3) State hop S_{c+1} = S_c + K_c^T V_c (not needed after the last
        // chunk of a segment whose successor starts from the scanned state).
        if (c + 1 < c1 || last_seg) state_hop<Cf>(Sacc, Vf, Ks, w, g, c16);
        __syncthreads();
    }

    if (last_seg) {
        float* Sout = S + bh * dkdv;
#pragma unroll
        for (int vw = 0; vw < Cf::NVW; ++vw) {
            const int v = 16 * (w + kWaves * vw) + c16;
#pragma unroll
            for (int dt = 0; dt < Cf::NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 16 * dt + 4 * g + r;
                    if (d < dk && v < dv) Sout[(int64_t)d * dv + v] = Sacc[vw][dt][r];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: planning and dispatch over (input type, chunk tile, head dim).
// ---------------------------------------------------------------------------
static int pad_dim(int x) { return x <= 32 ? 32 : (x <= 64 ? 64 : 128); }

void plan_prefill(PrefillPlan& p) {
    p.BH = p.B * p.H;
    p.D = pad_dim(p.dk > p.dv ? p.dk : p.dv);
    p.CT = pad_dim(p.C);
    p.n_c = p.T > 0 ? (p.T + p.C - 1) / p.C : 0;
    const int64_t want = p.n_c * p.BH;
    p.G = want > kTargetWalkers ? (want + kTargetWalkers - 1) / kTargetWalkers : 1;
    if (p.G > p.n_c) p.G = p.n_c > 0 ? p.n_c : 1;
    p.n_seg = p.n_c > 0 ? (p.n_c + p.G - 1) / p.G : 0;
    const int ve = p.dtype == LLA_BF16 ? 8 : 4;
    p.vec = (p.dk % ve == 0) && (p.dv % ve == 0);
}

template <typename T, int CT, int D>
static hipError_t launch_walk_t(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                                float* S, float* O, float* ws, hipStream_t st) {
    const int64_t grid = p.BH * p.n_seg;
    hipLaunchKernelGGL((k_chunk_walk<T, CT, D>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                       (const T*)Q, (const T*)K, (const T*)V, S, O, (const float*)ws, p.T, p.dk,
                       p.dv, p.C, p.G, p.n_seg, (int)p.vec);
    return hipGetLastError();
}

template <typename T, int CT, int D>
static hipError_t launch_seg_t(const PrefillPlan& p, const void* K, const void* V, float* ws,
                               hipStream_t st) {
    const int64_t grid = p.BH * (p.n_seg - 1);
    hipLaunchKernelGGL((k_segment_states<T, CT, D>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                       (const T*)K, (const T*)V, ws, p.T, p.dk, p.dv, p.C, p.G, p.n_seg,
                       (int)p.vec);
    return hipGetLastError();
}

// Calls F<T, CT, D>::run(args...) for the plan's padded sizes.
#define LLA_DISPATCH(FN, ...)                                                              \
    do {                                                                                   \
        if (p.dtype == LLA_BF16) {                                                         \
            if (p.CT == 32) {                                                              \
                if (p.D == 32) return FN<bf16, 32, 32>(__VA_ARGS__);                       \
                if (p.D == 64) return FN<bf16, 32, 64>(__VA_ARGS__);                       \
                return FN<bf16, 32, 128>(__VA_ARGS__);                                     \
            } else if (p.CT == 64) {                                                       \
                if (p.D == 32) return FN<bf16, 64, 32>(__VA_ARGS__);                       \
                if (p.D == 64) return FN<bf16, 64, 64>(__VA_ARGS__);                       \
                return FN<bf16, 64, 128>(__VA_ARGS__);                                     \
            } else {                                                                       \
                if (p.D == 32) return FN<bf16, 128, 32>(__VA_ARGS__);                      \
                if (p.D == 64) return FN<bf16, 128, 64>(__VA_ARGS__);                      \
                return FN<bf16, 128, 128>(__VA_ARGS__);                                    \
            }                                                                              \
        } else {                                                                           \
            if (p.CT == 32) {                                                              \
                if (p.D == 32) return FN<float, 32, 32>(__VA_ARGS__);                      \
                if (p.D == 64) return FN<float, 32, 64>(__VA_ARGS__);                      \
                return FN<float, 32, 128>(__VA_ARGS__);                                    \
            } else {                                                                       \
                if (p.D == 32) return FN<float, 64, 32>(__VA_ARGS__);                      \
                if (p.D == 64) return FN<float, 64, 64>(__VA_ARGS__);                      \
                return FN<float, 64, 128>(__VA_ARGS__);                                    \
            }                                                                              \
        }                                                                                  \
    } while (0)

hipError_t launch_chunk_walk(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                             float* S, float* O, float* ws, hipStream_t st) {
    if (p.n_c == 0) return hipSuccess;
    LLA_DISPATCH(launch_walk_t, p, Q, K, V, S, O, ws, st);
}

hipError_t launch_segment_states(const PrefillPlan& p, const void* K, const void* V, float* ws,
                                 hipStream_t st) {
    if (p.n_seg <= 1) return hipSuccess;
    LLA_DISPATCH(launch_seg_t, p, K, V, ws, st);
}

hipError_t launch_state_scan(const PrefillPlan& p, const float* S, float* ws, hipStream_t st) {
    if (p.n_seg <= 1) return hipSuccess;
    const int64_t dkdv = (int64_t)p.dk * p.dv;
    const int64_t per_block = (int64_t)kThreads * 4;
    const int64_t blocks_per_bh = (dkdv + per_block - 1) / per_block;
    hipLaunchKernelGGL(k_state_scan, dim3((unsigned)(p.BH * blocks_per_bh)), dim3(kThreads), 0, st,
                       S, ws, p.n_seg, dkdv, blocks_per_bh);
    return hipGetLastError();
}

}  // namespace lla
