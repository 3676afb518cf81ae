// lla_prefill.hip -- chunkwise-parallel causal linear-attention prefill for
// gfx950 (MI355X).
//
// Method (slide deck "Chunking, causality, and parallel prefill"): per chunk c
// of C tokens, O_c = tril(Q_c K_c^T) V_c + Q_c S_c and S_{c+1} = S_c + K_c^T V_c
// ("Split into chunks", "Causal triangle", "Incoming and outgoing state");
// only the chunk-to-chunk state hop is serial.
//
// Three kernels:
//   k_segment_states : per (b,h), segment of G chunks and block of value
//                      columns, the increment K_seg^T V_seg (fp32, matrix cores).
//   k_state_scan     : exclusive prefix over segments -> the state each
//                      segment starts from (the serial hop, one add per
//                      segment instead of one per chunk).
//   k_chunk_walk     : one workgroup per (b,h), segment and block of value
//                      columns walks its G chunks with the fp32 state slice
//                      in registers: scores on matrix cores, causal mask in
//                      registers, masked scores times V plus Q times the state
//                      (state split into bf16 high + low parts), then the
//                      state hop K_c^T V_c.
//
// Matrix-core layout (16x16 tiles, 32-deep steps): see lla::mma.  The score
// tile is computed transposed (keys as rows) so that a lane holds four
// consecutive key columns of one query row -- one 8-byte LDS write -- and the
// output tile is computed transposed (values as rows) so that a lane holds
// four consecutive output columns -- one 16-byte global store.  Operands that
// contract over time (K^T in the state hop, V everywhere) are read from the
// row-major LDS tiles with the gfx950 LDS transpose read (lla::lds_col).
#include "lla_device.h"
#include "lla_internal.h"

#include <type_traits>

namespace lla {

template <typename T, int CT_, int D_, int BV_, int NW_ = kWaves>
struct WalkCfg {
    static constexpr int CT = CT_, D = D_, BV = BV_;
    static constexpr int NW = NW_, NTH = NW * kWave;  // waves, threads per workgroup
    static constexpr bool BF = std::is_same<T, bf16>::value;
    // The state operand of Q S in natural depth order, so that Q is read in
    // 16-byte rows (see state_operand).  Chunks of 128 keep the interleaved
    // order: their walks have no registers to spare for the regrouping.
    static constexpr bool NATQ = BF && CT <= 64;
    // The masked scores P as a bf16 high + low pair (second tile right after
    // P), so that P V carries P to about 16 bits instead of bf16's 8: an
    // output dominated by one large score term then keeps fp32-like accuracy.
    // Chunks of 128 have no LDS to spare for the second tile.
    static constexpr bool SPLITP = BF && CT <= 64 && LLA_SPLIT_P;
    static constexpr int NP = SPLITP ? 2 : 1;  // P tiles
    // LDS row strides (elements), chosen for the 64 four-byte LDS banks:
    //  Q: 8 (mod 16) dwords with NATQ -- its 16-byte row reads, in the
    //     scores and in Q S, are conflict-free; else 4 (mod 8) dwords, for
    //     the 8-byte pairs of Q S;
    //  K, V: 8 (mod 16) dwords -- a transpose read by two 16-lane groups
    //     covers 8 consecutive rows x 32 bytes, on distinct banks;
    //  P: 4 (mod 8) dwords -- its 8-byte writes and reads are conflict-free.
    static constexpr int LQ = D + (NATQ ? 16 : (BF ? 8 : 4));
    static constexpr int LK = D + (BF ? 16 : 4);
    static constexpr int LV = BV + (BF ? 16 : 4);
    static constexpr int LP = CT + (BF ? 8 : 4);
    using LQL = PadLayout<LQ>;
    using LKL = PadLayout<LK>;
    using LVL = PadLayout<LV>;
    // One LDS buffer per workgroup: the Q, K, V and score tiles during the
    // walk; the fp32 state slice (D x BV, row stride SLD) before and after it.
    static constexpr int K_OFF = CT * LQ, V_OFF = K_OFF + CT * LK, P_OFF = V_OFF + CT * LV;
    static constexpr int SLD = BV + 4;
    static constexpr int STATE_BYTES = D * SLD * 4;
    static constexpr int WALK_BYTES = (P_OFF + NP * CT * LP) * (int)sizeof(T) > STATE_BYTES
                                          ? (P_OFF + NP * CT * LP) * (int)sizeof(T) : STATE_BYTES;
    static constexpr int SEG_TILES = (CT * LK + CT * LV) * (int)sizeof(T);
    static constexpr int SEG_BYTES = SEG_TILES > STATE_BYTES ? SEG_TILES : STATE_BYTES;
    static constexpr int NT = CT / 16;              // 16-row tiles per chunk
    static constexpr int NTS = CT / 32;             // 32-deep time steps per chunk
    static constexpr int NDT = D / 16;              // 16-wide tiles over the key dim
    static constexpr int NDS = D / 32;              // 32-deep steps over the key dim
    static constexpr int NVT = BV / 16;             // value tiles in the block
    static constexpr int NVW = (NVT + NW - 1) / NW;  // value tiles per wave
    static constexpr bool ALL_WAVES = NVT % NW == 0;  // every wave owns tiles
    static constexpr int NTRI = NT * (NT + 1) / 2;           // lower-triangle tiles
    using Fr = typename Frag<T>::type;
};

// ---- LDS operand reads -------------------------------------------------------

// 8 consecutive elements of one row (the depth index runs along the row).
__device__ __forceinline__ bf16x8 lds_row(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ f32x8 lds_row(const float* p) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// 4 + 4 elements of one row from two 8-byte aligned addresses.
__device__ __forceinline__ bf16x8 lds_row2(const bf16* p0, const bf16* p1) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 lds_row2(const float* p0, const float* p1) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p1);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Operand slice down one column of a row-major tile (row stride ld): lane
// (group g, column c16) gets, in slots s = 0..3 and 4..7, the elements
// M[row0 + 4g + s][col0 + c16] and M[row0 + 16 + 4g + (s - 4)][col0 + c16]
// -- the interleaved depth order used by every product that contracts over
// time.  bf16 uses the LDS transpose read: within a 16-lane group, lanes
// 4r..4r+3 address row r of a 4x16 block and lane i receives column i; the
// two groups that share an LDS pass then read 8 consecutive rows.
__device__ __forceinline__ bf16x8 lds_col(const bf16* base, int ld, int row0, int col0, int lane) {
    const int r = (lane >> 2) & 3, j = lane & 3, g = lane >> 4;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const bf16* p0 = base + (row0 + 4 * g + r) * ld + col0 + 4 * j;
    const bf16* p1 = p0 + 16 * ld;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<bf16*>(p0)));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<bf16*>(p1)));
    const bf16x4 ab = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
    return bf16x8{ab[0], ab[1], ab[2], ab[3], bb[0], bb[1], bb[2], bb[3]};
}
__device__ __forceinline__ f32x8 lds_col(const float* base, int ld, int row0, int col0, int lane) {
    const float* p = base + (row0 + 4 * (lane >> 4)) * ld + col0 + (lane & 15);
    f32x8 f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        f[s] = p[s * ld];
        f[4 + s] = p[(16 + s) * ld];
    }
    return f;
}

__device__ __forceinline__ void lds_store4(bf16* p, f32x4 x) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
}
__device__ __forceinline__ void lds_store4(float* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
}
// x = hi + lo, both rounded to bf16: hi to p_hi, lo to p_lo.
__device__ __forceinline__ void lds_store4_split(bf16* p_hi, bf16* p_lo, f32x4 x) {
    bf16x4 h, l;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float xr = x[r];
        const bf16 hr = to_bf16(xr);
        h[r] = hr;
        l[r] = to_bf16(xr - to_f32(hr));
    }
    *reinterpret_cast<bf16x4*>(p_hi) = h;
    *reinterpret_cast<bf16x4*>(p_lo) = l;
}

// ---- work mapping ---------------------------------------------------------------

// Workgroup id -> (line, value block), where a "line" is one (b,h,segment).
// Consecutive ids go round-robin over the 8 XCDs, so the value blocks of one
// line get ids congruent mod 8: they share an XCD and its L2, where the
// second block's Q and K reads hit.
__device__ __forceinline__ void split_id(int64_t id, int64_t n_lines, int n_vb, int64_t& line,
                                         int& vb) {
    const int64_t per = 8 * (int64_t)n_vb;
    const int64_t grp = id / per, off = id - grp * per;
    const int64_t r = min((int64_t)8, n_lines - 8 * grp);
    vb = (int)(off / r);
    line = 8 * grp + off % r;
}

// The value-column operand slices of a wave: V[32 ts + (time slot)][16 vt + c16].
template <typename Cf, typename T>
__device__ __forceinline__ void load_vfrags(typename Cf::Fr (&Vf)[Cf::NVW][Cf::NTS], const T* Vs,
                                            int w, int g, int lane) {
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) {
        const int vt = w + Cf::NW * vw;
#pragma unroll
        for (int ts = 0; ts < Cf::NTS; ++ts)
            if (Cf::ALL_WAVES || vt < Cf::NVT)
                Vf[vw][ts] = lds_col(Vs, Cf::LV, 32 * ts, 16 * vt, lane);
    }
}

// The fp32 state slice moves between global memory and registers through
// LDS: coalesced 16-byte global accesses on one side, the matrix-core
// accumulator layout (lane (g, c16) holds S[16 dt + 4g + r][16 vt + c16]) on
// the other.  Rows d >= dk and columns >= nv read as zero and are not written.
template <typename Cf>
__device__ __forceinline__ void state_gmem_to_lds(float* lds, const float* g, int dk, int dv,
                                                  int nv, int tid) {
    constexpr int VPR = Cf::BV / 4;
    if ((dv & 3) == 0) {
        for (int e = tid; e < Cf::D * VPR; e += Cf::NTH) {
            const int d = e / VPR, c = 4 * (e % VPR);
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (d < dk && c < nv) x = *reinterpret_cast<const f32x4*>(g + (int64_t)d * dv + c);
            *reinterpret_cast<f32x4*>(lds + d * Cf::SLD + c) = x;
        }
    } else {
        for (int e = tid; e < Cf::D * Cf::BV; e += Cf::NTH) {
            const int d = e / Cf::BV, c = e % Cf::BV;
            lds[d * Cf::SLD + c] = (d < dk && c < nv) ? g[(int64_t)d * dv + c] : 0.0f;
        }
    }
}
template <typename Cf>
__device__ __forceinline__ void state_lds_to_gmem(float* g, const float* lds, int dk, int dv,
                                                  int nv, int tid) {
    constexpr int VPR = Cf::BV / 4;
    if ((dv & 3) == 0) {
        for (int e = tid; e < Cf::D * VPR; e += Cf::NTH) {
            const int d = e / VPR, c = 4 * (e % VPR);
            if (d < dk && c < nv)
                *reinterpret_cast<f32x4*>(g + (int64_t)d * dv + c) =
                    *reinterpret_cast<const f32x4*>(lds + d * Cf::SLD + c);
        }
    } else {
        for (int e = tid; e < Cf::D * Cf::BV; e += Cf::NTH) {
            const int d = e / Cf::BV, c = e % Cf::BV;
            if (d < dk && c < nv) g[(int64_t)d * dv + c] = lds[d * Cf::SLD + c];
        }
    }
}
template <typename Cf>
__device__ __forceinline__ void state_lds_to_regs(f32x4 (&Sacc)[Cf::NVW][Cf::NDT], const float* lds,
                                                  int w, int g, int c16) {
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) {
        const int vt = (Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT) ? w + Cf::NW * vw : 0;
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sacc[vw][dt][r] = lds[(16 * dt + 4 * g + r) * Cf::SLD + 16 * vt + c16];
    }
}
template <typename Cf>
__device__ __forceinline__ void state_regs_to_lds(float* lds, const f32x4 (&Sacc)[Cf::NVW][Cf::NDT],
                                                  int w, int g, int c16) {
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) {
        if (!(Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT)) continue;
        const int vt = w + Cf::NW * vw;
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                lds[(16 * dt + 4 * g + r) * Cf::SLD + 16 * vt + c16] = Sacc[vw][dt][r];
    }
}

// The same moves straight between global memory and the accumulator layout,
// 4 bytes per lane per element: lane (g, c16) of wave w reads or writes
// S[16 dt + 4g + r][16 vt + c16], so one instruction covers four 64-byte row
// pieces.  Used where the LDS round trip (a 64 KB stage and two barriers)
// would sit on the critical path.  Rows >= dk and columns >= nv read as zero
// (the buffer range drops them) and are not written.
template <typename Cf>
__device__ __forceinline__ void state_gmem_to_regs(f32x4 (&Sacc)[Cf::NVW][Cf::NDT], const float* g_state,
                                                   int dk, int dv, int nv, int w, int g, int c16) {
    const rsrc_t rs = make_rsrc(g_state, (uint32_t)((int64_t)dk * dv * 4));
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) {
        const int col = 16 * (w + Cf::NW * vw) + c16;
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * dt + 4 * g + r;
                const uint32_t off = (row < dk && col < nv) ? (uint32_t)((row * dv + col) * 4) : kOutside;
                Sacc[vw][dt][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
            }
    }
}
template <typename Cf>
__device__ __forceinline__ void state_regs_to_gmem(float* g_state, const f32x4 (&Sacc)[Cf::NVW][Cf::NDT],
                                                   int dk, int dv, int w, int g, int c16) {
    const rsrc_t rs = make_rsrc(g_state, (uint32_t)((int64_t)dk * dv * 4));
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) {
        const int col = 16 * (w + Cf::NW * vw) + c16;
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * dt + 4 * g + r;
                const uint32_t off = (row < dk && col < dv) ? (uint32_t)((row * dv + col) * 4) : kOutside;
                // (the element goes through a scalar: this compiler bit-casts a
                // subscripted vector element as element 0)
                const float x = Sacc[vw][dt][r];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, off, 0, 0);
            }
    }
}

// State hop for the tiles a wave owns: S[:, value tile w + 4 vw] += K^T V,
// contracting over the CT rows (time) of the staged tiles.
template <typename Cf, typename T>
__device__ __forceinline__ void state_hop(f32x4 (&Sacc)[Cf::NVW][Cf::NDT],
                                          const typename Cf::Fr (&Vf)[Cf::NVW][Cf::NTS],
                                          const T* Ks, int w, int g, int lane) {
#pragma unroll
    for (int dt = 0; dt < Cf::NDT; ++dt) {
#pragma unroll
        for (int ts = 0; ts < Cf::NTS; ++ts) {
            const typename Cf::Fr kt = lds_col(Ks, Cf::LK, 32 * ts, 16 * dt, lane);
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
                if (Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT)
                    Sacc[vw][dt] = mma(kt, Vf[vw][ts], Sacc[vw][dt]);
        }
    }
}

// ---- the math of one chunk, shared by the walk kernels ---------------------------

// Masked scores of the chunk staged in Qs, Ks -> P (Ps), for the tiles wave w
// owns.  Every wave of the workgroup must call it; Ps is complete after the
// next barrier.
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};

// The score tiles wave w owns: triangle tiles e = w, w + NW, ... as (query
// tile it, key tile jt) pairs.  A wave short of tiles repeats the last one
// (computed, not stored).  Depends on the wave alone: built once per kernel.
template <typename Cf>
struct ScoreTiles {
    static constexpr int PW = (Cf::NTRI + Cf::NW - 1) / Cf::NW;
    int it[PW], jt[PW];
    bool own[PW];
    __device__ __forceinline__ explicit ScoreTiles(int w) {
#pragma unroll
        for (int m = 0; m < PW; ++m) {
            const int e0 = w + Cf::NW * m;
            const int e = e0 < Cf::NTRI ? e0 : Cf::NTRI - 1;
            int row = 0;
#pragma unroll
            for (int k = 1; k < Cf::NT; ++k) row += k * (k + 1) / 2 <= e;
            it[m] = row;
            jt[m] = e - row * (row + 1) / 2;
            own[m] = e0 < Cf::NTRI;
        }
    }
};

// `hook(ds)` runs after the matrix-core ops of depth step ds: a caller can
// place other work (global stores, loads) between the steps.
template <typename Cf, typename T, typename Hook = NoHook>
__device__ __forceinline__ void chunk_scores(const ScoreTiles<Cf>& st, const T* Qs, const T* Ks, T* Ps,
                                             int w, int g, int c16, const Hook& hook = Hook()) {
    // Scores of the kept triangle, computed transposed: tile (jt, it) holds
    // A^T = K_c Q_c^T, i.e. lane (g, c16) has A[i][j] for query
    // i = 16 it + c16 and keys j = 16 jt + 4g + r.  Entries with j > i are
    // masked in registers; the rest is rounded to the input type (P).
    // Wave w owns tiles w, w + NW, ... of the triangle and runs them as
    // independent accumulators (a wave short of tiles recomputes the last
    // one and does not store it), so the matrix-core latency overlaps.
    {
        constexpr int PW = ScoreTiles<Cf>::PW;
        const int* tit = st.it;
        const int* tjt = st.jt;
        f32x4 sacc[PW];
#pragma unroll
        for (int m = 0; m < PW; ++m) sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < Cf::NDS; ++ds) {
#pragma unroll
            for (int m = 0; m < PW; ++m)
                sacc[m] = mma(lds_row(Ks + (16 * tjt[m] + c16) * Cf::LK + 32 * ds + 8 * g),
                              lds_row(Qs + (16 * tit[m] + c16) * Cf::LQ + 32 * ds + 8 * g), sacc[m]);
            hook(ds);
        }
#pragma unroll
        for (int m = 0; m < PW; ++m) {
            if (!st.own[m]) continue;
            const int i = 16 * tit[m] + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * tjt[m] + 4 * g + r > i) sacc[m][r] = 0.0f;
            if constexpr (Cf::SPLITP)
                lds_store4_split(Ps + i * Cf::LP + 16 * tjt[m] + 4 * g,
                                 Ps + Cf::CT * Cf::LP + i * Cf::LP + 16 * tjt[m] + 4 * g, sacc[m]);
            else
                lds_store4(Ps + i * Cf::LP + 16 * tjt[m] + 4 * g, sacc[m]);
        }
    }
    // Tiles right of the diagonal that a 32-deep step still reads: zero.
    for (int it = 2 * w; it + 1 < Cf::NT; it += 2 * Cf::NW)
#pragma unroll
        for (int pt = 0; pt < Cf::NP; ++pt)
            lds_store4(Ps + pt * Cf::CT * Cf::LP + (16 * it + c16) * Cf::LP + 16 * (it + 1) + 4 * g,
                       f32x4{0.f, 0.f, 0.f, 0.f});
}

// One depth step of the state operand: value row c16 and eight depth slots.
// The lane holds depths {4g + r} of tile 2ds and {16 + 4g + r} of tile
// 2ds + 1 (the accumulator layout).  Without NATQ the operand uses exactly
// those slots, and Q is read to match in two 8-byte halves.  With NATQ they
// are regrouped with two lane swaps into the natural order, depths
// 8g .. 8g + 7, so that Q's slice is one 16-byte row read: 8-byte LDS reads
// run at half the rate of 16-byte ones.  The 32-lane swap trades lane groups
// {2, 3} of tile 2ds with groups {0, 1} of tile 2ds + 1; the 16-lane swap
// then trades the odd groups of the first with the even groups of the
// second.  bf16 inputs: S = hi + lo (lo is zero for fp32).
template <typename Cf>
__device__ __forceinline__ void state_operand(typename Cf::Fr& hi, typename Cf::Fr& lo,
                                              const f32x4 (&Sv)[Cf::NDT], int ds) {
    if constexpr (Cf::NATQ) {
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float fa = Sv[2 * ds][r], fb = Sv[2 * ds + 1][r];
            const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(fa), __float_as_uint(fb), false, false);
            const uint32_t a32 = p32[0], b32 = p32[1];
            const auto p16 = __builtin_amdgcn_permlane16_swap(a32, b32, false, false);
            const uint32_t a16 = p16[0], b16 = p16[1];
            x[r] = __uint_as_float(a16);
            x[4 + r] = __uint_as_float(b16);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16 h = to_bf16(x[s]);
            hi[s] = h;
            lo[s] = to_bf16(x[s] - to_f32(h));
        }
    } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float x = Sv[2 * ds + (s >> 2)][s & 3];
            if constexpr (Cf::BF) {
                const bf16 h = to_bf16(x);
                hi[s] = h;
                lo[s] = to_bf16(x - to_f32(h));
            } else {
                hi[s] = x;
            }
        }
    }
}

// O_c for the value tiles wave w owns: Oacc[it][vw] = (P V_c + Q_c S_c)^T,
// from P (Ps), the wave's V operand slices Vf, Q (Qs) and the state slice
// Sacc.  Oacc is overwritten.  The Q S part is software pipelined: the Q
// slices and the state operand of depth step ds + 1 are read and formed
// while the matrix-core ops of step ds run; `hook(ds)` runs after step ds.
template <typename Cf, typename T, typename Hook = NoHook>
__device__ __forceinline__ void chunk_output(f32x4 (&Oacc)[Cf::NT][Cf::NVW],
                                             const f32x4 (&Sacc)[Cf::NVW][Cf::NDT],
                                             const typename Cf::Fr (&Vf)[Cf::NVW][Cf::NTS],
                                             const T* Qs, const T* Ps, int w, int g, int c16,
                                             const Hook& hook = Hook()) {
    using Fr = typename Cf::Fr;
    auto q_slices = [&](Fr (&qb)[Cf::NT], int ds) {  // depth slots as in state_operand
#pragma unroll
        for (int it = 0; it < Cf::NT; ++it) {
            const int i = 16 * it + c16;
            if constexpr (Cf::NATQ)
                qb[it] = lds_row(Qs + i * Cf::LQ + 32 * ds + 8 * g);
            else
                qb[it] = lds_row2(Qs + i * Cf::LQ + 32 * ds + 4 * g, Qs + i * Cf::LQ + 32 * ds + 16 + 4 * g);
        }
    };
    auto owns = [&](int vw) { return Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT; };

    Fr qb[2][Cf::NT], Shi[2][Cf::NVW], Slo[2][Cf::NVW];
    q_slices(qb[0], 0);
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw) state_operand<Cf>(Shi[0][vw], Slo[0][vw], Sacc[vw], 0);

    // All query tiles of the chunk are accumulated side by side (depth
    // outer, tile inner), so consecutive matrix-core ops are independent.
#pragma unroll
    for (int it = 0; it < Cf::NT; ++it)
#pragma unroll
        for (int vw = 0; vw < Cf::NVW; ++vw) Oacc[it][vw] = f32x4{0.f, 0.f, 0.f, 0.f};
    // masked scores times values: a 32-deep time step ts reaches query
    // tiles it >= 2 ts (steps right of the diagonal are all zero)
#pragma unroll
    for (int ts = 0; ts < Cf::NTS; ++ts) {
#pragma unroll
        for (int it = 2 * ts; it < Cf::NT; ++it) {
            const int i = 16 * it + c16;
            const Fr pb = lds_row2(Ps + i * Cf::LP + 32 * ts + 4 * g,
                                   Ps + i * Cf::LP + 32 * ts + 16 + 4 * g);
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
                if (owns(vw)) Oacc[it][vw] = mma(Vf[vw][ts], pb, Oacc[it][vw]);
            if constexpr (Cf::SPLITP) {  // the low part of P
                const T* Pl = Ps + Cf::CT * Cf::LP;
                const Fr pl = lds_row2(Pl + i * Cf::LP + 32 * ts + 4 * g, Pl + i * Cf::LP + 32 * ts + 16 + 4 * g);
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw)
                    if (owns(vw)) Oacc[it][vw] = mma(Vf[vw][ts], pl, Oacc[it][vw]);
            }
        }
    }
    // incoming state read: Q_c S_c
#pragma unroll
    for (int ds = 0; ds < Cf::NDS; ++ds) {
        const int cur = ds & 1, nxt = cur ^ 1;
        if (ds + 1 < Cf::NDS) {
            q_slices(qb[nxt], ds + 1);
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
                state_operand<Cf>(Shi[nxt][vw], Slo[nxt][vw], Sacc[vw], ds + 1);
        }
#pragma unroll
        for (int vw = 0; vw < Cf::NVW; ++vw) {
            if (!owns(vw)) continue;
#pragma unroll
            for (int it = 0; it < Cf::NT; ++it) Oacc[it][vw] = mma(Shi[cur][vw], qb[cur][it], Oacc[it][vw]);
            if constexpr (Cf::BF) {
#pragma unroll
                for (int it = 0; it < Cf::NT; ++it) Oacc[it][vw] = mma(Slo[cur][vw], qb[cur][it], Oacc[it][vw]);
            }
        }
        hook(ds);
    }
}

// ---------------------------------------------------------------------------
// Phase 1: per-segment state increments K_seg^T V_seg -> ws slot seg + 1,
// one workgroup per (b,h), segment (all but the last) and value block.
// ---------------------------------------------------------------------------
template <typename In, int CT, int D, int BV, bool VEC, int NW = kWaves>
__global__ __launch_bounds__(NW * kWave) void k_segment_states(
    const In* __restrict__ K, const In* __restrict__ V, float* __restrict__ ws, int64_t T_len,
    int dk, int dv, int C, int64_t G, int64_t n_seg, int n_vb) {
    using T = typename Compute<In>::type;
    using Cf = WalkCfg<T, CT, D, BV, NW>;
    using Fr = typename Cf::Fr;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::SEG_BYTES];
    T* Ks = reinterpret_cast<T*>(smem);
    T* Vs = Ks + CT * Cf::LK;
    float* Sst = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t nsm1 = n_seg - 1;
    int64_t line;
    int vb;
    split_id(blockIdx.x, (int64_t)(gridDim.x / n_vb), n_vb, line, vb);
    const int64_t bh = line / nsm1, seg = line - bh * nsm1;
    const int v0 = vb * BV;
    const int nv = min(BV, dv - v0);
    const int64_t n_c = (T_len + C - 1) / C;
    const int64_t c0 = seg * G, c1 = min(n_c, c0 + G);
    const In* Kb = K + bh * T_len * dk;
    const In* Vb = V + bh * T_len * dv + v0;

    f32x4 Sacc[Cf::NVW][Cf::NDT];
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt) Sacc[vw][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto rows_of = [&](int64_t c) { return (int)min((int64_t)C, T_len - c * C); };
    if constexpr (VEC) {
        // The loop is bound by memory latency, not by its math: keep PF
        // chunks of loads in flight (one register set per chunk, used round
        // robin; the loop is unrolled by PF so the sets are static).
        constexpr int PF = 2;
        Tile<T, CT, D, typename Cf::LKL, Cf::NTH, In> tk[PF];
        Tile<T, CT, BV, typename Cf::LVL, Cf::NTH, In> tv[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            tk[u].init(dk, dk, tid);
            tv[u].init(dv, nv, tid);
            if (c0 + u < c1) {
                tk[u].gather(Kb + (c0 + u) * C * dk, dk, rows_of(c0 + u));
                tv[u].gather(Vb + (c0 + u) * C * dv, dv, rows_of(c0 + u));
            }
        }
        for (int64_t c = c0; c < c1; c += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int64_t cc = c + u;
                if (cc >= c1) break;
                tk[u].scatter(Ks, tid);
                tv[u].scatter(Vs, tid);
                __syncthreads();
                if (cc + PF < c1) {
                    tk[u].gather(Kb + (cc + PF) * C * dk, dk, rows_of(cc + PF));
                    tv[u].gather(Vb + (cc + PF) * C * dv, dv, rows_of(cc + PF));
                }
                Fr Vf[Cf::NVW][Cf::NTS];
                load_vfrags<Cf>(Vf, Vs, w, g, lane);
                state_hop<Cf>(Sacc, Vf, Ks, w, g, lane);
                __syncthreads();
            }
        }
    } else {
        for (int64_t c = c0; c < c1; ++c) {
            Tile<T, CT, D, typename Cf::LKL, Cf::NTH, In>::load_scalar(Kb + c * C * dk, dk, rows_of(c), dk, Ks, tid);
            Tile<T, CT, BV, typename Cf::LVL, Cf::NTH, In>::load_scalar(Vb + c * C * dv, dv, rows_of(c), nv, Vs, tid);
            __syncthreads();
            Fr Vf[Cf::NVW][Cf::NTS];
            load_vfrags<Cf>(Vf, Vs, w, g, lane);
            state_hop<Cf>(Sacc, Vf, Ks, w, g, lane);
            __syncthreads();
        }
    }

    // (the loop ended with a barrier: the tiles are free)
    state_regs_to_lds<Cf>(Sst, Sacc, w, g, c16);
    __syncthreads();
    state_lds_to_gmem<Cf>(ws + (bh * n_seg + seg + 1) * (int64_t)dk * dv + v0, Sst, dk, dv, nv, tid);
}

// ---------------------------------------------------------------------------
// Phase 2: slot 0 = S_0, slot s = S_0 + sum_{s' < s} increment(s').
// One thread per 4 consecutive state elements of one (b,h).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_state_scan(const float* __restrict__ S,
                                                         float* __restrict__ ws, int64_t n_seg,
                                                         int64_t dkdv, int64_t blocks_per_bh,
                                                         int zero_start) {
    const int64_t bh = blockIdx.x / blocks_per_bh;
    const int64_t e = ((blockIdx.x % blocks_per_bh) * kThreads + threadIdx.x) * 4;
    if (e >= dkdv) return;
    float* slot = ws + bh * n_seg * dkdv + e;
    const float* s0 = S + bh * dkdv + e;
    if (e + 4 <= dkdv && (dkdv & 3) == 0) {
        // S_0 and the first U increments are loaded together (one memory
        // round trip), then summed in segment order.  The first batch always
        // runs, so slot 0 receives S_0 even for a single segment (grouped
        // heads read their start state from there).
        constexpr int U = 16;  // loads in flight per thread (segments per batch)
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (!zero_start) acc = *reinterpret_cast<const f32x4*>(s0);
        for (int64_t s = 1; s < n_seg || s == 1; s += U) {
            f32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s + u < n_seg) x[u] = *reinterpret_cast<const f32x4*>(slot + (s + u) * dkdv);
            if (s == 1) *reinterpret_cast<f32x4*>(slot) = acc;
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
            float acc = zero_start ? 0.0f : s0[j];
            slot[j] = acc;
            for (int64_t s = 1; s < n_seg; ++s) {
                acc += slot[s * dkdv + j];
                slot[s * dkdv + j] = acc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Phase 3: the chunk walk.  One workgroup per (b,h), segment and block of BV
// value columns; four waves; the fp32 state slice S[:, block] lives in
// registers, split over the waves by value tiles (wave w owns tiles w, w+4..).
// ---------------------------------------------------------------------------
// Writes a chunk's output tiles held by a wave: Oacc[it][vw] holds
// O[t0 + 16 it + c16][v0 + 16 vt + 4g + r], r = 0..3 (vt = w + 4 vw).  The
// vector path stores through a buffer descriptor that ends at the chunk's
// last valid row, so rows past it are dropped without a branch.
template <typename Cf, bool VEC>
__device__ __forceinline__ void store_out(float* Ob, const f32x4 (&Oacc)[Cf::NT][Cf::NVW], int64_t t0,
                                          int nrows, int nv, int dv, int w, int g, int c16) {
    if constexpr (VEC) {
        const rsrc_t rs = make_rsrc(Ob + t0 * dv, (uint32_t)(nrows * dv * 4));
#pragma unroll
        for (int it = 0; it < Cf::NT; ++it) {
            const int i = 16 * it + c16;
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw) {
                const int v = 16 * (w + Cf::NW * vw) + 4 * g;
                if (!(Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT)) continue;
                const uint32_t off = v < nv ? (uint32_t)((i * dv + v) * 4) : kOutside;
                buf_store16(rs, off, Oacc[it][vw]);
            }
        }
    } else {
#pragma unroll
        for (int it = 0; it < Cf::NT; ++it) {
            const int i = 16 * it + c16;
            if (i >= nrows) continue;
            float* orow = Ob + (t0 + i) * dv;
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw) {
                const int v = 16 * (w + Cf::NW * vw) + 4 * g;
                if (!(Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT) || v >= nv) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (v + r < nv) orow[v + r] = Oacc[it][vw][r];
            }
        }
    }
}

template <typename In, int CT, int D, int BV, bool VEC, int NW = kWaves>
__global__ __launch_bounds__(NW * kWave) void k_chunk_walk(
    const In* __restrict__ Q, const In* __restrict__ K, const In* __restrict__ V,
    float* __restrict__ S, float* __restrict__ O, const float* __restrict__ ws, int64_t T_len,
    int dk, int dv, int C, int64_t G, int64_t n_seg, int n_vb, int group, int zero_start) {
    using T = typename Compute<In>::type;
    using Cf = WalkCfg<T, CT, D, BV, NW>;
    using Fr = typename Cf::Fr;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::WALK_BYTES];
    T* Qs = reinterpret_cast<T*>(smem);
    T* Ks = Qs + Cf::K_OFF;
    T* Vs = Qs + Cf::V_OFF;
    T* Ps = Qs + Cf::P_OFF;
    float* Sst = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int64_t line;
    int vb;
    split_id(blockIdx.x, (int64_t)(gridDim.x / n_vb), n_vb, line, vb);
    // line = (query head, segment); the query heads of a group share the
    // key/value head bh = bq / group: its K, V and states
    const int64_t bq = line / n_seg, seg = line - bq * n_seg, bh = bq / group;
    const ScoreTiles<Cf> stiles(w);
    const int v0 = vb * BV;
    const int nv = min(BV, dv - v0);  // valid columns of this block
    const int64_t n_c = (T_len + C - 1) / C;
    const int64_t c0 = seg * G, c1 = min(n_c, c0 + G);
    const bool last_seg = seg == n_seg - 1;
    const int64_t dkdv = (int64_t)dk * dv;
    const In* Qb = Q + bq * T_len * dk;
    const In* Kb = K + bh * T_len * dk;
    const In* Vb = V + bh * T_len * dv + v0;
    float* Ob = O + bq * T_len * dv + v0;

    // Incoming state of this segment, columns [v0, v0 + nv).
    // (zero_start without a workspace: S_0 = 0, S is not read -- columns
    // past `nv` read as zero)
    const float* Sin = (ws == nullptr ? S + bh * dkdv : ws + (bh * n_seg + seg) * dkdv) + v0;
    f32x4 Sacc[Cf::NVW][Cf::NDT];
    state_gmem_to_lds<Cf>(Sst, Sin, dk, dv, (ws == nullptr && zero_start) ? 0 : nv, tid);
    __syncthreads();
    state_lds_to_regs<Cf>(Sacc, Sst, w, g, c16);
    __syncthreads();  // the state area is reused by the tiles

    using TQ = Tile<T, CT, D, typename Cf::LQL, Cf::NTH, In>;
    using TK = Tile<T, CT, D, typename Cf::LKL, Cf::NTH, In>;
    using TV = Tile<T, CT, BV, typename Cf::LVL, Cf::NTH, In>;
    TQ tq;
    TK tk;
    TV tv;
    auto rows_of = [&](int64_t c) { return (int)min((int64_t)C, T_len - c * C); };
    if constexpr (VEC) {
        tq.init(dk, dk, tid);
        tk.init(dk, dk, tid);
        tv.init(dv, nv, tid);
        tq.gather(Qb + c0 * C * dk, dk, rows_of(c0));
        tk.gather(Kb + c0 * C * dk, dk, rows_of(c0));
        tv.gather(Vb + c0 * C * dv, dv, rows_of(c0));
    }

    // A chunk's outputs stay in registers until the next chunk has started:
    // the wait for the next tiles' loads then never includes stores issued
    // late in the previous chunk (loads and stores share one counter).
    f32x4 Oacc[Cf::NT][Cf::NVW];
    int64_t t_prev = 0;
    int n_prev = 0;

    for (int64_t c = c0; c < c1; ++c) {
        const int nrows = rows_of(c);
        const int64_t t0 = c * C;
        if constexpr (VEC) {
            tq.scatter(Qs, tid);
            tk.scatter(Ks, tid);
            tv.scatter(Vs, tid);
        } else {
            TQ::load_scalar(Qb + t0 * dk, dk, nrows, dk, Qs, tid);
            TK::load_scalar(Kb + t0 * dk, dk, nrows, dk, Ks, tid);
            TV::load_scalar(Vb + t0 * dv, dv, nrows, nv, Vs, tid);
        }
        __syncthreads();
        if (c > c0) store_out<Cf, VEC>(Ob, Oacc, t_prev, n_prev, nv, dv, w, g, c16);
        if constexpr (VEC) {
            if (c + 1 < c1) {  // next chunk's loads fly during this chunk's math
                const int nr = rows_of(c + 1);
                tq.gather(Qb + (t0 + C) * dk, dk, nr);
                tk.gather(Kb + (t0 + C) * dk, dk, nr);
                tv.gather(Vb + (t0 + C) * dv, dv, nr);
            }
        }

        chunk_scores<Cf>(stiles, Qs, Ks, Ps, w, g, c16);
        __syncthreads();

        // (2) Output, transposed: O^T tile (vt, it) = V^T P^T + S^T Q^T.
        Fr Vf[Cf::NVW][Cf::NTS];
        load_vfrags<Cf>(Vf, Vs, w, g, lane);

        chunk_output<Cf>(Oacc, Sacc, Vf, Qs, Ps, w, g, c16);
        t_prev = t0;
        n_prev = nrows;

        // State hop S_{c+1} = S_c + K_c^T V_c (not needed after the last
        // chunk of a segment whose successor starts from the scanned state).
        if (c + 1 < c1 || last_seg) state_hop<Cf>(Sacc, Vf, Ks, w, g, lane);
        __syncthreads();
    }
    if (c1 > c0) store_out<Cf, VEC>(Ob, Oacc, t_prev, n_prev, nv, dv, w, g, c16);

    if (last_seg && bq % group == 0) {  // one writer per group (the loop ended with a barrier)
        state_regs_to_lds<Cf>(Sst, Sacc, w, g, c16);
        __syncthreads();
        state_lds_to_gmem<Cf>(S + bh * dkdv + v0, Sst, dk, dv, nv, tid);
    }
}

// ---------------------------------------------------------------------------
// Phase 3, wide form for d = 128 bf16 (or FP8, staged as bf16) inputs and
// chunks of up to 64 tokens:
// one workgroup of eight waves per (b,h) and segment covers all 128 value
// columns (wave w owns value tile w), so the score triangle is computed and
// the Q, K tiles are loaded once per chunk.  Q, K, V are double buffered in
// LDS: while chunk c is computed from one buffer, chunk c+1 is written into
// the other from registers loaded one chunk earlier and the loads of chunk
// c+2 are issued -- two barriers per chunk, none of them behind a load.
// ---------------------------------------------------------------------------
#ifndef LLA_WIDE_WAVES
#define LLA_WIDE_WAVES 8
#endif
constexpr int kWideWaves = LLA_WIDE_WAVES;  // waves of the wide walk (value tiles per wave: 8 / waves)

template <int CT>
struct WideCfg : WalkCfg<bf16, CT, 128, 128, kWideWaves> {
    using Base = WalkCfg<bf16, CT, 128, 128, kWideWaves>;
    static constexpr int BUF = Base::P_OFF;  // elements of one Q, K, V buffer
    // two Q, K, V buffers and P; the state moves between global memory and
    // registers directly, so it takes no LDS
    static constexpr int BYTES = (2 * BUF + Base::NP * CT * Base::LP) * 2;
};

template <int CT, typename In>
__global__ __launch_bounds__(kWideWaves * kWave) void k_chunk_walk_wide(
    const In* __restrict__ Q, const In* __restrict__ K, const In* __restrict__ V,
    float* __restrict__ S, float* __restrict__ O, const float* __restrict__ ws, int64_t T_len,
    int dk, int dv, int C, int64_t G, int64_t n_seg, int group, int zero_start) {
    using Cf = WideCfg<CT>;
    using Fr = typename Cf::Fr;
    constexpr int NTH = Cf::NTH;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::BYTES];
    bf16* const buf = reinterpret_cast<bf16*>(smem);
    bf16* const Ps = buf + 2 * Cf::BUF;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t line = blockIdx.x;
    const ScoreTiles<Cf> stiles(w);
    // line = (query head, segment); the group's key/value head is bq / group
    const int64_t bq = line / n_seg, seg = line - bq * n_seg, bh = bq / group;
    const int64_t n_c = (T_len + C - 1) / C;
    const int64_t c0 = seg * G, c1 = min(n_c, c0 + G);
    const bool last_seg = seg == n_seg - 1;
    const int64_t dkdv = (int64_t)dk * dv;
    const In* Qb = Q + bq * T_len * dk;
    const In* Kb = K + bh * T_len * dk;
    const In* Vb = V + bh * T_len * dv;
    float* Ob = O + bq * T_len * dv;
    auto rows_of = [&](int64_t c) { return c < c1 ? (int)min((int64_t)C, T_len - c * C) : 0; };

    // The first chunk's tile loads, then the incoming state straight into
    // the accumulator registers: the first chunk's scores need only the
    // tiles, so the state arrives while they run (loads complete in order).
    // (zero_start without a workspace: S_0 = 0 -- no column is read)
    Tile<bf16, CT, 128, typename Cf::LQL, NTH, In> tq;
    Tile<bf16, CT, 128, typename Cf::LKL, NTH, In> tk;
    Tile<bf16, CT, 128, typename Cf::LVL, NTH, In> tv;
    tq.init(dk, dk, tid);
    tk.init(dk, dk, tid);
    tv.init(dv, dv, tid);
    tq.gather(Qb + c0 * C * dk, dk, rows_of(c0));
    tk.gather(Kb + c0 * C * dk, dk, rows_of(c0));
    tv.gather(Vb + c0 * C * dv, dv, rows_of(c0));
    const float* Sin = ws == nullptr ? S + bh * dkdv : ws + (bh * n_seg + seg) * dkdv;
    f32x4 Sacc[Cf::NVW][Cf::NDT];
    state_gmem_to_regs<Cf>(Sacc, Sin, dk, dv, (ws == nullptr && zero_start) ? 0 : dv, w, g, c16);
    tq.scatter(buf, tid);
    tk.scatter(buf + Cf::K_OFF, tid);
    tv.scatter(buf + Cf::V_OFF, tid);
    tq.gather(Qb + (c0 + 1) * C * dk, dk, rows_of(c0 + 1));
    tk.gather(Kb + (c0 + 1) * C * dk, dk, rows_of(c0 + 1));
    tv.gather(Vb + (c0 + 1) * C * dv, dv, rows_of(c0 + 1));
    __syncthreads();

    // A chunk's outputs are stored during the next chunk (see k_chunk_walk).
    f32x4 Oacc[Cf::NT][Cf::NVW];
#pragma unroll
    for (int it = 0; it < Cf::NT; ++it)
#pragma unroll
        for (int vw = 0; vw < Cf::NVW; ++vw) Oacc[it][vw] = f32x4{0.f, 0.f, 0.f, 0.f};
    int64_t t_prev = 0;
    int n_prev = 0;

    for (int64_t c = c0; c < c1; ++c) {
        const int b = (int)((c - c0) & 1);
        const bf16* Qs = buf + b * Cf::BUF;
        const bf16* Ks = Qs + Cf::K_OFF;
        const bf16* Vs = Qs + Cf::V_OFF;
        bf16* nxt = buf + (1 - b) * Cf::BUF;

        // The global traffic of a chunk is spread over its math, so that
        // the eight waves do not queue their memory instructions at once:
        // the previous chunk's output tiles are stored one per depth step of
        // the scores, the loads of chunk c + 2 go between the depth steps of
        // the output.
        const rsrc_t rso = make_rsrc(Ob + t_prev * dv, (uint32_t)(n_prev * dv * 4));
        chunk_scores<Cf>(stiles, Qs, Ks, Ps, w, g, c16, [&](int ds) {
            if (ds < Cf::NT) {
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw) {
                    const int vcol = 16 * (w + Cf::NW * vw) + 4 * g;
                    const uint32_t off = vcol < dv ? (uint32_t)(((16 * ds + c16) * dv + vcol) * 4) : kOutside;
                    buf_store16(rso, off, Oacc[ds][vw]);
                }
            }
        });
        // The next chunk into the free buffer (its last readers finished
        // before the previous barrier).
        if (c + 1 < c1) {
            tq.scatter(nxt, tid);
            tk.scatter(nxt + Cf::K_OFF, tid);
            tv.scatter(nxt + Cf::V_OFF, tid);
        }
        __syncthreads();  // P complete

        const int64_t t2 = (c + 2) * C;
        const int n2 = rows_of(c + 2);
        const rsrc_t rq = tq.source(Qb + t2 * dk, dk, n2), rk = tk.source(Kb + t2 * dk, dk, n2),
                     rv = tv.source(Vb + t2 * dv, dv, n2);
        Fr Vf[Cf::NVW][Cf::NTS];
        load_vfrags<Cf>(Vf, Vs, w, g, lane);
        chunk_output<Cf>(Oacc, Sacc, Vf, Qs, Ps, w, g, c16, [&](int ds) {
#pragma unroll
            for (int n = 0; n < decltype(tq)::NPT; ++n) {
                if (ds == 0) tq.load(rq, n);
                if (ds == 1) tk.load(rk, n);
                if (ds == 2) tv.load(rv, n);
            }
        });
        t_prev = c * C;
        n_prev = rows_of(c);
        if (c + 1 < c1 || last_seg) state_hop<Cf>(Sacc, Vf, Ks, w, g, lane);
        __syncthreads();  // this buffer and P free; the next buffer visible
    }
    store_out<Cf, true>(Ob, Oacc, t_prev, n_prev, dv, dv, w, g, c16);

    if (last_seg && bq % group == 0)  // one writer per group
        state_regs_to_gmem<Cf>(S + bh * dkdv, Sacc, dk, dv, w, g, c16);
}

// ---------------------------------------------------------------------------
// Phase 1, wide form for d = 128 bf16 (or FP8) inputs and chunks of up to 64 tokens:
// one workgroup of eight waves per (b,h) and segment (all but the last)
// covers all 128 value columns, so K is loaded once.  The K, V tiles are
// double buffered: chunk c + 1 is written into the free buffer while chunk
// c is reduced, and the loads of chunk c + 2 go between the matrix-core
// steps -- one barrier per chunk.
// ---------------------------------------------------------------------------
template <int CT>
struct SegWideCfg : WalkCfg<bf16, CT, 128, 128, 8> {
    using Base = WalkCfg<bf16, CT, 128, 128, 8>;
    static constexpr int V_AT = CT * Base::LK;             // V tile inside a buffer
    static constexpr int BUF = V_AT + CT * Base::LV;       // elements of one K, V buffer
    static constexpr int TILE_BYTES = 2 * BUF * 2;
    static constexpr int BYTES = TILE_BYTES > Base::STATE_BYTES ? TILE_BYTES : Base::STATE_BYTES;
};

template <int CT, typename In>
__global__ __launch_bounds__(512) void k_segment_states_wide(const In* __restrict__ K,
                                                             const In* __restrict__ V,
                                                             float* __restrict__ ws, int64_t T_len,
                                                             int dk, int dv, int C, int64_t G,
                                                             int64_t n_seg) {
    using Cf = SegWideCfg<CT>;
    using Fr = typename Cf::Fr;
    constexpr int NTH = Cf::NTH;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::BYTES];
    bf16* const buf = reinterpret_cast<bf16*>(smem);
    float* const Sst = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t nsm1 = n_seg - 1;
    const int64_t bh = blockIdx.x / nsm1, seg = blockIdx.x - bh * nsm1;
    const int64_t n_c = (T_len + C - 1) / C;
    const int64_t c0 = seg * G, c1 = min(n_c, c0 + G);
    const In* Kb = K + bh * T_len * dk;
    const In* Vb = V + bh * T_len * dv;
    auto rows_of = [&](int64_t c) { return c < c1 ? (int)min((int64_t)C, T_len - c * C) : 0; };

    f32x4 Sacc[Cf::NVW][Cf::NDT];
#pragma unroll
    for (int dt = 0; dt < Cf::NDT; ++dt) Sacc[0][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // PF register sets, used round robin (the loop is unrolled by PF so the
    // sets are static): the loads of chunk c + PF are issued while chunk c
    // is reduced, PF - 1 chunks ahead of their use.  Deeper rings measured
    // slower (more registers, two workgroups per CU either way).
    constexpr int PF = 2;
    using TK = Tile<bf16, CT, 128, typename Cf::LKL, NTH, In>;
    TK tk[PF];
    Tile<bf16, CT, 128, typename Cf::LVL, NTH, In> tv[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        tk[u].init(dk, dk, tid);
        tv[u].init(dv, dv, tid);
        tk[u].gather(Kb + (c0 + u) * C * dk, dk, rows_of(c0 + u));
        tv[u].gather(Vb + (c0 + u) * C * dv, dv, rows_of(c0 + u));
    }
    tk[0].scatter(buf, tid);
    tv[0].scatter(buf + Cf::V_AT, tid);
    __syncthreads();

    for (int64_t cb = c0; cb < c1; cb += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int64_t c = cb + u;
            if (c >= c1) break;
            const int b = (int)((c - c0) & 1);
            const bf16* Ks = buf + b * Cf::BUF;
            const bf16* Vs = Ks + Cf::V_AT;
            bf16* nxt = buf + (1 - b) * Cf::BUF;
            const int un = (u + 1) % PF;  // the set holding chunk c + 1 (static after unrolling)
            if (c + 1 < c1) {  // the free buffer's last readers passed the previous barrier
                tk[un].scatter(nxt, tid);
                tv[un].scatter(nxt + Cf::V_AT, tid);
            }
            // set u held chunk c, written to LDS one chunk ago: reload it
            const int64_t tn = (c + PF) * C;
            const int nn = rows_of(c + PF);
            const rsrc_t rk = tk[u].source(Kb + tn * dk, dk, nn), rv = tv[u].source(Vb + tn * dv, dv, nn);

            Fr Vf[Cf::NVW][Cf::NTS];
            load_vfrags<Cf>(Vf, Vs, w, g, lane);
#pragma unroll
            for (int dt = 0; dt < Cf::NDT; ++dt) {
#pragma unroll
                for (int ts = 0; ts < Cf::NTS; ++ts)
                    Sacc[0][dt] = mma(lds_col(Ks, Cf::LK, 32 * ts, 16 * dt, lane), Vf[0][ts], Sacc[0][dt]);
#pragma unroll
                for (int n = 0; n < TK::NPT; ++n) {
                    if (dt == 1) tk[u].load(rk, n);
                    if (dt == 3) tv[u].load(rv, n);
                }
            }
            __syncthreads();  // this buffer free; the next one visible
        }
    }

    // (the loop ended with a barrier: the tiles are free)
    state_regs_to_lds<Cf>(Sst, Sacc, w, g, c16);
    __syncthreads();
    state_lds_to_gmem<Cf>(ws + (bh * n_seg + seg + 1) * (int64_t)dk * dv, Sst, dk, dv, dv, tid);
}

// ---------------------------------------------------------------------------
// Host side: planning and dispatch over (input type, chunk tile, head dim).
// ---------------------------------------------------------------------------
static int pad_dim(int x) { return x <= 32 ? 32 : (x <= 64 ? 64 : 128); }

void plan_prefill(PrefillPlan& p) {
    if (p.Hkv == 0) p.Hkv = p.H;
    p.group = (int)(p.H / p.Hkv);
    p.BH = p.B * p.Hkv;   // key/value heads: states, segment pass, scan
    p.BHq = p.B * p.H;    // query heads: the walk
    p.D = pad_dim(p.dk > p.dv ? p.dk : p.dv);
    p.CT = pad_dim(p.C);
    p.BV = p.D > 64 ? 64 : p.D;
    p.n_vb = p.D / p.BV;
    p.n_c = p.T > 0 ? (p.T + p.C - 1) / p.C : 0;
    const int64_t want = p.n_c * p.BHq * p.n_vb;
    p.G = want > kTargetWalkers ? (want + kTargetWalkers - 1) / kTargetWalkers : 1;
    if (p.G > p.n_c) p.G = p.n_c > 0 ? p.n_c : 1;
    p.n_seg = p.n_c > 0 ? (p.n_c + p.G - 1) / p.G : 0;
    // a walk reads its starting state from the workspace when there are
    // several segments, or several query heads per state (the group's walks
    // must not read S while one of them writes S_T)
    p.use_ws = p.n_seg > 1 || p.group > 1;
    const int ve = p.dtype == LLA_FP8_E4M3 ? 16 : (p.dtype == LLA_BF16 ? 8 : 4);  // per 16 bytes
    p.vec = (p.dk % ve == 0) && (p.dv % ve == 0);
}

// In: the input element type (bf16, FP8 or fp32); the matrix cores run on
// Compute<In>::type.
template <typename In, int CT, int D>
static hipError_t launch_walk_t(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                                float* S, float* O, float* ws, hipStream_t st) {
    using T = typename Compute<In>::type;
    if constexpr (std::is_same<T, bf16>::value && D == 128 && CT <= 64) {
        if (p.vec) {  // one eight-wave workgroup per (b,h) and segment
            hipLaunchKernelGGL((k_chunk_walk_wide<CT, In>), dim3((unsigned)(p.BHq * p.n_seg)), dim3(kWideWaves * kWave), 0, st,
                               (const In*)Q, (const In*)K, (const In*)V, S, O,
                               (const float*)(p.use_ws ? ws : nullptr), p.T, p.dk, p.dv, p.C, p.G,
                               p.n_seg, p.group, (int)p.zero_start);
            return hipGetLastError();
        }
    }
    if constexpr (std::is_same<T, bf16>::value && D == 128 && CT == 128) {
        if (p.vec) {  // chunks of 128: one single-buffered eight-wave workgroup per (b,h) and segment
            hipLaunchKernelGGL((k_chunk_walk<In, 128, 128, 128, true, 8>), dim3((unsigned)(p.BHq * p.n_seg)),
                               dim3(8 * kWave), 0, st, (const In*)Q, (const In*)K, (const In*)V, S, O,
                               (const float*)(p.use_ws ? ws : nullptr), p.T, p.dk, p.dv, p.C, p.G,
                               p.n_seg, 1, p.group, (int)p.zero_start);
            return hipGetLastError();
        }
    }
    constexpr int BV = D > 64 ? 64 : D;
    const int64_t grid = p.BHq * p.n_seg * p.n_vb;
    const float* wsr = p.use_ws ? ws : nullptr;
    if (p.vec)
        hipLaunchKernelGGL((k_chunk_walk<In, CT, D, BV, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                           st, (const In*)Q, (const In*)K, (const In*)V, S, O, wsr, p.T,
                           p.dk, p.dv, p.C, p.G, p.n_seg, p.n_vb, p.group, (int)p.zero_start);
    else
        hipLaunchKernelGGL((k_chunk_walk<In, CT, D, BV, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                           st, (const In*)Q, (const In*)K, (const In*)V, S, O, wsr, p.T,
                           p.dk, p.dv, p.C, p.G, p.n_seg, p.n_vb, p.group, (int)p.zero_start);
    return hipGetLastError();
}

template <typename In, int CT, int D>
static hipError_t launch_seg_t(const PrefillPlan& p, const void* K, const void* V, float* ws,
                               hipStream_t st) {
    using T = typename Compute<In>::type;
    if constexpr (std::is_same<T, bf16>::value && D == 128 && CT <= 64) {
        if (p.vec) {  // one eight-wave workgroup per (b,h) and segment
            hipLaunchKernelGGL((k_segment_states_wide<CT, In>), dim3((unsigned)(p.BH * (p.n_seg - 1))),
                               dim3(512), 0, st, (const In*)K, (const In*)V, ws, p.T, p.dk, p.dv,
                               p.C, p.G, p.n_seg);
            return hipGetLastError();
        }
    }
    if constexpr (std::is_same<T, bf16>::value && D == 128 && CT == 128) {
        if (p.vec) {  // chunks of 128: one eight-wave workgroup per (b,h) and segment
            hipLaunchKernelGGL((k_segment_states<In, 128, 128, 128, true, 8>),
                               dim3((unsigned)(p.BH * (p.n_seg - 1))), dim3(8 * kWave), 0, st,
                               (const In*)K, (const In*)V, ws, p.T, p.dk, p.dv, p.C, p.G, p.n_seg, 1);
            return hipGetLastError();
        }
    }
    constexpr int BV = D > 64 ? 64 : D;
    const int64_t grid = p.BH * (p.n_seg - 1) * p.n_vb;
    if (p.vec)
        hipLaunchKernelGGL((k_segment_states<In, CT, D, BV, true>), dim3((unsigned)grid), dim3(kThreads),
                           0, st, (const In*)K, (const In*)V, ws, p.T, p.dk, p.dv, p.C, p.G, p.n_seg,
                           p.n_vb);
    else
        hipLaunchKernelGGL((k_segment_states<In, CT, D, BV, false>), dim3((unsigned)grid), dim3(kThreads),
                           0, st, (const In*)K, (const In*)V, ws, p.T, p.dk, p.dv, p.C, p.G, p.n_seg,
                           p.n_vb);
    return hipGetLastError();
}

// Calls FN<In, CT, D>(args...) for the plan's input type and padded sizes.
#define LLA_DISPATCH(FN, ...)                                                              \
    do {                                                                                   \
        if (p.dtype == LLA_FP8_E4M3) {                                                     \
            if (p.CT == 32) {                                                              \
                if (p.D == 32) return FN<fp8e4m3, 32, 32>(__VA_ARGS__);                    \
                if (p.D == 64) return FN<fp8e4m3, 32, 64>(__VA_ARGS__);                    \
                return FN<fp8e4m3, 32, 128>(__VA_ARGS__);                                  \
            } else if (p.CT == 64) {                                                       \
                if (p.D == 32) return FN<fp8e4m3, 64, 32>(__VA_ARGS__);                    \
                if (p.D == 64) return FN<fp8e4m3, 64, 64>(__VA_ARGS__);                    \
                return FN<fp8e4m3, 64, 128>(__VA_ARGS__);                                  \
            } else {                                                                       \
                if (p.D == 32) return FN<fp8e4m3, 128, 32>(__VA_ARGS__);                   \
                if (p.D == 64) return FN<fp8e4m3, 128, 64>(__VA_ARGS__);                   \
                return FN<fp8e4m3, 128, 128>(__VA_ARGS__);                                 \
            }                                                                              \
        } else if (p.dtype == LLA_BF16) {                                                  \
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
    if (!p.use_ws) return hipSuccess;
    const int64_t dkdv = (int64_t)p.dk * p.dv;
    const int64_t per_block = (int64_t)kThreads * 4;
    const int64_t blocks_per_bh = (dkdv + per_block - 1) / per_block;
    hipLaunchKernelGGL(k_state_scan, dim3((unsigned)(p.BH * blocks_per_bh)), dim3(kThreads), 0, st,
                       S, ws, p.n_seg, dkdv, blocks_per_bh, (int)p.zero_start);
    return hipGetLastError();
}

}  // namespace lla
