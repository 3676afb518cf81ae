// lla_prefill.hip -- chunkwise-parallel causal linear-attention prefill for
// gfx950 (MI355X).
//
// Method (slide deck "Chunking, causality, and parallel prefill"): per chunk c
// of C tokens, O_c = tril(Q_c K_c^T) V_c + Q_c S_c and S_{c+1} = S_c + K_c^T V_c
// ("Split into chunks", "Causal triangle", "Incoming and outgoing state");
// only the chunk-to-chunk state hop is serial.  Chunks of more than 64
// tokens run as two sub-chunks (see lla_plan.cpp), so tiles are 32 or 64 rows.
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
    static_assert(CT_ == 32 || CT_ == 64, "chunk tiles are 32 or 64 rows (longer chunks run as two sub-chunks)");
    // The state operand of Q S in natural depth order, so that Q is read in
    // 16-byte rows (see state_operand).
    static constexpr bool NATQ = BF;
    // The masked scores P as a bf16 high + low pair (second tile right after
    // P), so that P V carries P to about 16 bits instead of bf16's 8: an
    // output dominated by one large score term then keeps fp32-like accuracy.
    static constexpr bool SPLITP = BF && LLA_SPLIT_P;
    static constexpr int NP = SPLITP ? 2 : 1;  // P tiles
    // LDS row strides (elements), chosen for the 64 four-byte LDS banks:
    //  Q: 8 (mod 16) dwords with NATQ -- its 16-byte row reads, in the
    //     scores and in Q S, are conflict-free; else 4 (mod 8) dwords, for
    //     the 8-byte pairs of Q S;
    //  K, V: 8 (mod 16) dwords -- a transpose read by two 16-lane groups
    //     covers 8 consecutive rows x 32 bytes, on distinct banks;
    //  P: bf16, 8 (mod 16) dwords, like K and V, for its 16-byte reads (its
    //     columns are stored in the order of those reads, see p_col); fp32,
    //     4 (mod 8) dwords -- its 8-byte writes and reads are conflict-free.
    static constexpr int LQ = D + (NATQ ? 16 : (BF ? 8 : 4));
    static constexpr int LK = D + (BF ? 16 : 4);
    static constexpr int LV = BV + (BF ? 16 : 4);
    // P is stored as far as P V reads it: query tile it (rows 16 it ..
    // 16 it + 15) needs the columns of the 32-deep time steps 0 .. it / 2,
    // 32 (it / 2 + 1) of them.  Tiles it and NT - 1 - it need 32 (NT / 2 + 1)
    // columns together, so each such pair shares 16 rows of one stride:
    // tile it < NT / 2 from column 0, its partner right after it.  At
    // C = 64 a P tile is 3,584 elements instead of the 5,120 of the padded
    // square; one row stride keeps every tile's lane offset the same.
    static constexpr int PPAD = BF ? 16 : 4;
    static constexpr int PLD = 32 * (CT / 32 + 1) + PPAD;  // elements per row
    __device__ __host__ static constexpr int p_row0(int it) { return 16 * (it < CT / 32 ? it : CT / 16 - 1 - it); }
    __device__ __host__ static constexpr int p_col0(int it) {
        return it < CT / 32 ? 0 : 32 * ((CT / 16 - 1 - it) / 2 + 1);
    }
    // Where column col of P sits in its row.  bf16: each 32-column block
    // holds its columns in the depth order of the P V operand, which the
    // transpose read of V fixes (slots 0..3 of lane group g: columns
    // 4g .. 4g + 3, slots 4..7: 16 + 4g .. 16 + 4g + 3), so that a lane's
    // operand is one 16-byte read instead of two 8-byte ones; the scores are
    // still written 4 columns (8 bytes) at a time.  fp32: natural order.
    __device__ __host__ static constexpr int p_col(int col) {
        return BF ? (col & ~31) + 8 * ((col & 15) >> 2) + 4 * ((col >> 4) & 1) + (col & 3) : col;
    }
    // element (row 16 it + r, column col) of P
    __device__ __host__ static constexpr int p_at(int it, int r, int col) {
        return (p_row0(it) + r) * PLD + p_col0(it) + p_col(col);
    }
    static constexpr int PG = BF ? 8 : 4;  // p_col(c + 4g) - p_col(c) for c a multiple of 16, per g
    static constexpr int P_ELEMS = CT / 2 * PLD;  // one P tile
    using LQL = PadLayout<LQ>;
    using LKL = PadLayout<LK>;
    using LVL = PadLayout<LV>;
    // One LDS buffer per workgroup: the Q, K, V and score tiles during the
    // walk; the fp32 state slice (D x BV, row stride SLD) before and after it.
    static constexpr int K_OFF = CT * LQ, V_OFF = K_OFF + CT * LK, P_OFF = V_OFF + CT * LV;
    static constexpr int SLD = BV + 4;
    static constexpr int STATE_BYTES = D * SLD * 4;
    static constexpr int WALK_BYTES = (P_OFF + NP * P_ELEMS) * (int)sizeof(T) > STATE_BYTES
                                          ? (P_OFF + NP * P_ELEMS) * (int)sizeof(T) : STATE_BYTES;
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

// Workgroup id -> work unit such that units u, u + 1, ... share an XCD:
// ids go round-robin over the 8 XCDs, so XCD x takes the ids congruent to x
// mod 8 and receives a contiguous range of units (a bijection on [0, n)).
// The XCD (XCC) the calling wave runs on: hardware register XCC_ID, bits 0-3.
__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u; }

__device__ __forceinline__ int64_t xcd_major(int64_t id, int64_t n) {
    const int64_t x = id & 7, k = id >> 3, q = n >> 3, r = n & 7;
    return x * q + min(x, r) + k;
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
// No gate: chunk_scores keeps the masked scores as they are, chunk_output
// adds Q S unscaled (see DecayGate and DecayRows for the gated walk).
struct NoGate {};

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
// `group` > 0: query row i is token i / group of a group of query heads
// (see k_tokens_grouped), so key j is kept while j <= i / group.
// `gate(x, i, j0)` (gated walk) scales the masked scores x[r] of query i and
// keys j0 + r before they are stored.
template <typename Cf, typename T, typename Hook = NoHook, typename Gate = NoGate>
__device__ __forceinline__ void chunk_scores(const ScoreTiles<Cf>& st, const T* Qs, const T* Ks, T* Ps,
                                             int w, int g, int c16, const Hook& hook = Hook(),
                                             int group = 0, const Gate& gate = Gate()) {
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
            const int last = group > 0 ? i / group : i;  // the last key row i reads
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * tjt[m] + 4 * g + r > last) sacc[m][r] = 0.0f;
            if constexpr (!std::is_same<Gate, NoGate>::value) gate(sacc[m], i, 16 * tjt[m] + 4 * g);
            // the lane's part of the address, recomputed per chunk rather
            // than one live register per tile
            const int at = opaque(c16 * Cf::PLD + Cf::PG * g) + Cf::p_at(tit[m], 0, 16 * tjt[m]);
            if constexpr (Cf::SPLITP)
                lds_store4_split(Ps + at, Ps + Cf::P_ELEMS + at, sacc[m]);
            else
                lds_store4(Ps + at, sacc[m]);
        }
    }
    // Tiles right of the diagonal that a 32-deep step still reads: zero.
    for (int it = 2 * w; it + 1 < Cf::NT; it += 2 * Cf::NW)
#pragma unroll
        for (int pt = 0; pt < Cf::NP; ++pt)
            lds_store4(Ps + pt * Cf::P_ELEMS + opaque(c16 * Cf::PLD + Cf::PG * g) + Cf::p_at(it, 0, 16 * (it + 1)),
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
// `rows(it)` (gated walk): the factor of query row 16 it + c16's Q S part,
// which is then accumulated apart and added, scaled, after P V.
template <typename Cf, typename T, typename Hook = NoHook, typename RowScale = NoGate>
__device__ __forceinline__ void chunk_output(f32x4 (&Oacc)[Cf::NT][Cf::NVW],
                                             const f32x4 (&Sacc)[Cf::NVW][Cf::NDT],
                                             const typename Cf::Fr (&Vf)[Cf::NVW][Cf::NTS],
                                             const T* Qs, const T* Ps, int w, int g, int c16,
                                             const Hook& hook = Hook(), const RowScale& rows = RowScale()) {
    using Fr = typename Cf::Fr;
    constexpr bool SCALED = !std::is_same<RowScale, NoGate>::value;
    f32x4 Oqs[SCALED ? Cf::NT : 1][Cf::NVW];  // Q S apart (gated walk only)
    auto qs_acc = [&](int it, int vw) -> f32x4& {
        if constexpr (SCALED) return Oqs[it][vw];
        else return Oacc[it][vw];
    };
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

    // The first depth step's Q slices and state operand are read ahead of P V.
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
            const int at = Cf::p_at(it, c16, 32 * ts + 4 * g);
            auto p_operand = [&](const T* base) -> Fr {
                if constexpr (Cf::BF)
                    return lds_row(base + at);  // slots in storage order (p_col)
                else
                    return lds_row2(base + at, base + at + 16);
            };
            const Fr pb = p_operand(Ps);
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
                if (owns(vw)) Oacc[it][vw] = mma(Vf[vw][ts], pb, Oacc[it][vw]);
            if constexpr (Cf::SPLITP) {  // the low part of P
                const Fr pl = p_operand(Ps + Cf::P_ELEMS);
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw)
                    if (owns(vw)) Oacc[it][vw] = mma(Vf[vw][ts], pl, Oacc[it][vw]);
            }
        }
    }
    // incoming state read: Q_c S_c
    if constexpr (SCALED) {
#pragma unroll
        for (int it = 0; it < Cf::NT; ++it)
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw) qs_acc(it, vw) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
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
            for (int it = 0; it < Cf::NT; ++it) qs_acc(it, vw) = mma(Shi[cur][vw], qb[cur][it], qs_acc(it, vw));
            if constexpr (Cf::BF) {
#pragma unroll
                for (int it = 0; it < Cf::NT; ++it) qs_acc(it, vw) = mma(Slo[cur][vw], qb[cur][it], qs_acc(it, vw));
            }
        }
        hook(ds);
    }
    if constexpr (SCALED) {
#pragma unroll
        for (int it = 0; it < Cf::NT; ++it) {
            const float f = rows(it);
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
                for (int r = 0; r < 4; ++r) Oacc[it][vw][r] = fmaf(f, Oqs[it][vw][r], Oacc[it][vw][r]);
        }
    }
}

// ---------------------------------------------------------------------------
// Gated (decayed) state: S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, one
// gate g_t per (b,h) and token.  The slide deck cites the chunkwise form of
// gated linear attention ("Boundary, evidence, and sources") but gives no
// gate; this is the plainest decay, a scalar applied to the previous state
// before the token's update (g = 1: the walk above).  Gates are taken in
// [2^-126, 1]: g <= 0 (and NaN) acts as 2^-126, g > 1 as 1.
// Per chunk, with b_t = sum_{l <= t} log2 g_l over the chunk's rows (rows past
// the last count 0) and B = b_{CT-1}, the chunk form is
//     O_i     = sum_{j <= i} 2^{b_i - b_j} (q_i . k_j) v_j + 2^{b_i} q_i S_c
//     S_{c+1} = 2^B S_c + sum_j 2^{B - b_j} k_j v_j^T
// and every factor is at most 1.  The masked scores are scaled in fp32 before
// their bf16 high + low split; Q S is accumulated apart and added scaled in
// fp32; the hop takes V scaled by 2^{B - b_j} as a high + low pair.  So the
// numerics are the ungated walk's.  A segment's total decay (the sum of its
// chunks' B) goes to the workspace after the states, and the scan is
// P_{s+1} = 2^{L_s} P_s + increment_s.
// ---------------------------------------------------------------------------

// A chunk's decay table, 3 CT floats: D[t] = b_t, D[CT + t] = 2^{B - b_t}
// (the hop's factor of row t), D[2 CT + t] = 2^{b_t} (the incoming-state
// factor of query row t).  exp2 and log2 are the hardware instructions
// (about 1 ulp): arguments are at most 0, and results below 2^-126 only
// scale away terms that are already negligible.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave 0: a chunk's decay table from the gate g of row `lane` (1 past the
// chunk's rows).
template <int CT>
__device__ __forceinline__ void chunk_decay(float* D, float g, int lane) {
    auto log2g = [](float x) { return fminf(fmaxf(__builtin_amdgcn_logf(x), -126.0f), 0.0f); };
    auto scan = [&](float a) {
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const float y = __shfl_up(a, d, kWave);
            if (lane >= d) a += y;
        }
        return a;
    };
    static_assert(CT <= kWave, "one gate per lane");
    const float a = scan(log2g(g));
    const float B = __shfl(a, CT - 1, kWave);
    if (lane < CT) {
        D[lane] = a;
        D[CT + lane] = hw_exp2(B - a);
        D[2 * CT + lane] = hw_exp2(a);
    }
}

// Masked score (query i, keys j0 .. j0 + 3) times 2^{b_i - b_j} (masked
// entries are zero and stay zero: the factor is clamped to at most 1).
struct DecayGate {
    const float* Bs;  // the decay table
    __device__ __forceinline__ void operator()(f32x4& x, int i, int j0) const {
        const float bi = Bs[i];
        const f32x4 bj = *reinterpret_cast<const f32x4*>(Bs + j0);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = x[r] * hw_exp2(fminf(bi - bj[r], 0.0f));
    }
};
// The factor 2^{b_i} of query row i = 16 it + c16's incoming-state term.
template <int CT>
struct DecayRows {
    const float* Bs;  // the decay table
    int c16;
    __device__ __forceinline__ float operator()(int it) const { return Bs[2 * CT + 16 * it + c16]; }
};

// Gated state hop: S = 2^B S + K^T (2^{B - b} V), V's time slots as in
// load_vfrags (slot s of lane group g: time 32 ts + 4g + s, then 32 ts + 16 +
// 4g + s - 4).
template <typename Cf, typename T>
__device__ __forceinline__ void state_hop_gated(f32x4 (&Sacc)[Cf::NVW][Cf::NDT],
                                                const typename Cf::Fr (&Vf)[Cf::NVW][Cf::NTS],
                                                const T* Ks, const float* Bs, int w, int g, int lane) {
    using Fr = typename Cf::Fr;
    const float dS = Bs[3 * Cf::CT - 1];  // 2^B
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[vw][dt][r] = Sacc[vw][dt][r] * dS;
    Fr Vh[Cf::NVW][Cf::NTS], Vl[Cf::NVW][Cf::NTS];
#pragma unroll
    for (int ts = 0; ts < Cf::NTS; ++ts) {
        const f32x4 h0 = *reinterpret_cast<const f32x4*>(Bs + Cf::CT + 32 * ts + 4 * g);
        const f32x4 h1 = *reinterpret_cast<const f32x4*>(Bs + Cf::CT + 32 * ts + 16 + 4 * g);
        const float h[8] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
        for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float x = to_f32(Vf[vw][ts][s]) * h[s];
                if constexpr (Cf::BF) {
                    const bf16 hi = to_bf16(x);
                    Vh[vw][ts][s] = hi;
                    Vl[vw][ts][s] = to_bf16(x - to_f32(hi));
                } else {
                    Vh[vw][ts][s] = x;
                }
            }
    }
#pragma unroll
    for (int dt = 0; dt < Cf::NDT; ++dt) {
#pragma unroll
        for (int ts = 0; ts < Cf::NTS; ++ts) {
            const Fr kt = lds_col(Ks, Cf::LK, 32 * ts, 16 * dt, lane);
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw) {
                if (!(Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT)) continue;
                Sacc[vw][dt] = mma(kt, Vh[vw][ts], Sacc[vw][dt]);
                if constexpr (Cf::BF) Sacc[vw][dt] = mma(kt, Vl[vw][ts], Sacc[vw][dt]);
            }
        }
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
        for (int vw = 0; vw < Cf::NVW; ++vw) {
            const int v = 16 * (w + Cf::NW * vw) + 4 * g;
            if (!(Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT)) continue;
            // row c16 of every query tile: one lane offset, plus the tile's
            // first row (kOutside plus it stays outside)
            const uint32_t off = v < nv ? (uint32_t)((c16 * dv + v) * 4) : kOutside;
#pragma unroll
            for (int it = 0; it < Cf::NT; ++it)
                buf_store16(rs, opaque(off) + (uint32_t)(16 * it * dv * 4), Oacc[it][vw]);
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

// PREFIX: the walk of a fresh prompt or a verify pass (S is not both read
// and written) with few chunks before its last segment.  Instead of reading
// its start state from the workspace, each workgroup sums the earlier
// segments' K^T V itself: every segment's sum from zero over its chunks
// (the segment pass's products, in its order), each added to S_0 in segment
// order (the scan's additions) -- so the bits of the three phases, in one
// launch.  The lines of a query head are given workgroup ids that share an
// XCD, so the K and V rows they all read come from one L2.
template <typename In, int CT, int D, int BV, bool VEC, int NW = kWaves, bool PREFIX = false>
__global__ __launch_bounds__(NW * kWave) void k_chunk_walk(
    const In* __restrict__ Q, const In* __restrict__ K, const In* __restrict__ V,
    float* __restrict__ S, float* __restrict__ O, const float* __restrict__ ws, int64_t T_len,
    int dk, int dv, int C, int64_t G, int64_t n_seg, int n_vb, int group, int zero_start, int keep,
    float* __restrict__ pub, unsigned long long* __restrict__ flags, unsigned long long token,
    uint64_t wait_ticks) {
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
    if constexpr (PREFIX) {
        const int64_t u = xcd_major(blockIdx.x, gridDim.x);  // (line, value block), line-major
        line = u / n_vb;
        vb = (int)(u - line * n_vb);
    } else {
        split_id(blockIdx.x, (int64_t)(gridDim.x / n_vb), n_vb, line, vb);
    }
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
    // The first chunk's tiles: loaded into registers now (with PREFIX, their
    // round trip overlaps the earlier segments' sums), staged at the walk.
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
    if constexpr (PREFIX) {
        // The segments before this one, each summed from zero over its G
        // chunks (all full: only a sequence's last chunk is short, and it
        // lies in the last segment) and then added to S in segment order.
        f32x4 Inc[Cf::NVW][Cf::NDT];
        // Segments [ja, jb) summed in order: each one's Inc = sum over its
        // chunks of K_c^T V_c, from zero, in chunk order (the segment pass's
        // products); then, if `add`, S += Inc at the segment's end (the
        // scan's additions).  One ring of loads runs across the whole range.
        auto sum_segments = [&](int64_t ja, int64_t jb, bool add) {
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
                for (int dt = 0; dt < Cf::NDT; ++dt) Inc[vw][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int64_t a = ja * G, b = jb * G;
            int64_t left = G;  // chunks of the current segment still to sum
            auto hop = [&]() {  // the next chunk in order, staged in Ks, Vs
                Fr Vf[Cf::NVW][Cf::NTS];
                load_vfrags<Cf>(Vf, Vs, w, g, lane);
                state_hop<Cf>(Inc, Vf, Ks, w, g, lane);
                if (--left == 0 && add) {  // a segment's sum is complete
                    left = G;
#pragma unroll
                    for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
                        for (int dt = 0; dt < Cf::NDT; ++dt) {
                            Sacc[vw][dt] += Inc[vw][dt];
                            Inc[vw][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        }
                }
            };
            if constexpr (VEC) {
                constexpr int PF = 2;  // chunks of loads in flight (register sets used round robin)
                TK pk[PF];
                TV pv[PF];
#pragma unroll
                for (int u = 0; u < PF; ++u) {
                    pk[u].init(dk, dk, tid);
                    pv[u].init(dv, nv, tid);
                    if (a + u < b) {
                        pk[u].gather(Kb + (a + u) * C * dk, dk, C);
                        pv[u].gather(Vb + (a + u) * C * dv, dv, C);
                    }
                }
                for (int64_t c = a; c < b; c += PF) {
#pragma unroll
                    for (int u = 0; u < PF; ++u) {
                        const int64_t cc = c + u;
                        if (cc >= b) break;
                        pk[u].scatter(Ks, tid);
                        pv[u].scatter(Vs, tid);
                        __syncthreads();
                        if (cc + PF < b) {
                            pk[u].gather(Kb + (cc + PF) * C * dk, dk, C);
                            pv[u].gather(Vb + (cc + PF) * C * dv, dv, C);
                        }
                        hop();
                        __syncthreads();
                    }
                }
            } else {
                for (int64_t c = a; c < b; ++c) {
                    TK::load_scalar(Kb + c * C * dk, dk, C, dk, Ks, tid);
                    TV::load_scalar(Vb + c * C * dv, dv, C, nv, Vs, tid);
                    __syncthreads();
                    hop();
                    __syncthreads();
                }
            }
        };
        // Published sums (pub != null): every segment but the last sums its
        // own chunks first and stores the sum where the later segments of its
        // key/value head read it (one writer per group), so that a walk
        // reads an earlier segment's sum instead of summing it again.  A slot
        // holds one workgroup's Inc in register order ((w, vw, dt), then lane,
        // then the 4 rows): 16-byte accesses, no LDS stage.
        // The hand-over goes through the L2 of one XCD, which all its compute
        // units share (their vector caches write through to it, and a kernel
        // starts with them invalidated): the writer's stores are complete
        // in L2 before its flag is set, and a reader uses a slot only if its
        // flag names the reader's own XCD -- this call's token xor the
        // writer's XCD id.  Flags are device-scope atomics (one coherent value
        // for all XCDs), so no cache of another XCD is ever trusted and no
        // L2 is written back or invalidated.  A slot written on another XCD,
        // or not flagged by the deadline (wait_ticks of the 100 MHz real-time
        // counter after the first poll), is summed by the reader itself:
        // the same products in the same order, so the bits do not depend on
        // which happens, and no wait outlasts the deadline.
        constexpr int SLOT = Cf::NW * Cf::NVW * Cf::NDT * 256;  // floats per (segment, value block)
        auto slot_at = [&](int64_t j, int vw, int dt) {
            return pub + ((bh * n_seg + j) * n_vb + vb) * SLOT + (((w * Cf::NVW + vw) * Cf::NDT + dt) * 64 + lane) * 4;
        };
        auto flag_at = [&](int64_t j) { return flags + (bh * n_seg + j) * n_vb + vb; };
        const unsigned long long mine = token ^ (unsigned long long)xcc_id();
        if (pub != nullptr && !last_seg && bq % group == 0) {
            sum_segments(seg, seg + 1, false);  // (the sum stays in Inc)
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
                for (int dt = 0; dt < Cf::NDT; ++dt)
                    if (Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT)
                        *reinterpret_cast<f32x4*>(slot_at(seg, vw, dt)) = Inc[vw][dt];
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);  // this wave's stores acknowledged by L2
            __syncthreads();
            if (tid == 0) __hip_atomic_store(flag_at(seg), mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // Wave 0 decides, for the whole workgroup (the sums use barriers),
        // which earlier segments to read: lane j polls segment j's flag until
        // it names this XCD, names another one, or the deadline passes.
        __shared__ uint64_t use_sh;
        if (w == 0) {
            uint64_t use = 0;
            if (pub != nullptr && seg > 0) {
                const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + wait_ticks;
                const bool mine_lane = lane < seg;
                bool here = false, settled = !mine_lane;
                for (;;) {
                    if (!settled) {
                        const unsigned long long f =
                            __hip_atomic_load(flag_at(lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        here = f == mine;
                        settled = here || (f ^ token) < 16;  // flagged on this XCD or another one
                    }
                    if (__ballot(!settled) == 0 || __builtin_amdgcn_s_memrealtime() > deadline) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                use = __ballot(here);
            }
            if (lane == 0) use_sh = use;
        }
        __syncthreads();
        const uint64_t use = use_sh;  // (the same value in every lane)
        // Segments in order: a run of published ones is loaded up to eight
        // at a time (one memory round trip), a run of the others is summed
        // here with one ring of loads; each segment's sum is added to S in
        // segment order either way.
        auto published = [&](int64_t j) { return j < 64 && ((use >> j) & 1u); };
        constexpr int GRP = 8;
        for (int64_t j = 0; j < seg;) {
            if (!published(j)) {
                int64_t r = j + 1;
                while (r < seg && !published(r)) ++r;
                sum_segments(j, r, true);
                j = r;
                continue;
            }
            f32x4 Ld[GRP][Cf::NVW][Cf::NDT];
            int n = 0;
#pragma unroll
            for (int u = 0; u < GRP; ++u) {
                const bool from_slot = j + u < seg && published(j + u) && n == u;
                if (from_slot) ++n;
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
                    for (int dt = 0; dt < Cf::NDT; ++dt)
                        Ld[u][vw][dt] = (from_slot && (Cf::ALL_WAVES || w + Cf::NW * vw < Cf::NVT))
                                            ? *reinterpret_cast<const f32x4*>(slot_at(j + u, vw, dt))
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < GRP; ++u) {
                if (u >= n) break;
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
                    for (int dt = 0; dt < Cf::NDT; ++dt) Sacc[vw][dt] += Ld[u][vw][dt];
            }
            j += n;
        }
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
        // chunk of a segment whose successor starts from the scanned state,
        // nor after the last one when S_T is not kept).
        if (c + 1 < c1 || (last_seg && !keep)) state_hop<Cf>(Sacc, Vf, Ks, w, g, lane);
        __syncthreads();
    }
    if (c1 > c0) store_out<Cf, VEC>(Ob, Oacc, t_prev, n_prev, nv, dv, w, g, c16);

    // S_T: one writer per group (the loop ended with a barrier); none for a
    // verify pass, which leaves S as it was
    if (last_seg && bq % group == 0 && !keep) {
        state_regs_to_lds<Cf>(Sst, Sacc, w, g, c16);
        __syncthreads();
        state_lds_to_gmem<Cf>(S + bh * dkdv + v0, Sst, dk, dv, nv, tid);
    }
}

// ---------------------------------------------------------------------------
// Short continuations with shared-state heads, on the matrix cores.  For a
// key/value head with state S_0, T <= 16 new tokens and G query heads
// (T G <= 64), every output is
//     o_t^(g) = S_0^T q_t^(g) + sum_{s <= t} (q_t^(g) . k_s) v_s,
// which is one chunk of the walk: the T G query rows, ordered token-major
// (row r = t G + g), against the T key and value rows (rows past T are
// zero), with key s kept for row r while s <= r / G -- every kept entry lies
// in the walk's lower-triangle tiles.  So the chunk's helpers run unchanged:
// scores and mask (chunk_scores with the group's mask), O = P V + Q S_0
// (chunk_output), then S_T = S_0 + K^T V (state_hop).  For d = 64 (this
// kernel) one workgroup per key/value head, one value tile per wave, so that
// several workgroups share a compute unit and one's state loads overlap
// another's arithmetic; d = 128 takes the persistent k_tokens_grouped_pipe
// below.
// S enters Q S and P enters P V as bf16 high + low pairs, as in the walk, so
// integers are exact under the walk's bounds and floats carry the walk's
// error; the outputs are not the bits of T decode steps (the verify pass of
// speculative decoding keeps k_decode_tokens for that).
// q, o: [key/value head][g][T][D] (the group's query heads are consecutive);
// k, v: [key/value head][T][D]; S: [key/value head][D][D].
// ---------------------------------------------------------------------------

// Rows of a tile staged from global memory: row r < nrows comes from
// src(r) (D elements, 16-byte aligned), later rows are zero.  FP8 inputs are
// decoded to bf16 on the way.
template <typename In, int D, int LD, int ROWS, int NTH, typename Src>
__device__ __forceinline__ void stage_rows(bf16* lds, int nrows, const Src& src, int tid) {
    constexpr int VE = Vec<In>::n;  // input elements per 16-byte load
    constexpr int VPR = D / VE;
    for (int e = tid; e < ROWS * VPR; e += NTH) {
        const int row = e / VPR, cv = e % VPR;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row < nrows) x = *reinterpret_cast<const u32x4*>(src(row) + cv * VE);
        bf16* dst = lds + row * LD + cv * VE;
        if constexpr (sizeof(In) == 2) {
            *reinterpret_cast<u32x4*>(dst) = x;
        } else {  // 16 FP8 values -> two 8-element bf16 vectors
            uint32_t y[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) fp8x4_to_bf16(x[i], y[2 * i], y[2 * i + 1]);
            *reinterpret_cast<u32x4*>(dst) = u32x4{y[0], y[1], y[2], y[3]};
            *reinterpret_cast<u32x4*>(dst + 8) = u32x4{y[4], y[5], y[6], y[7]};
        }
    }
}

template <typename In, int D, int BV, int NW>
__global__ __launch_bounds__(NW * kWave) void k_tokens_grouped(
    const In* __restrict__ Q, const In* __restrict__ K, const In* __restrict__ V, float* __restrict__ S,
    float* __restrict__ O, int T, int G, int zero_start) {
    using Cf = WalkCfg<bf16, 64, D, BV, NW>;
    using Fr = typename Cf::Fr;
    constexpr int NTH = Cf::NTH;
    static_assert(Cf::ALL_WAVES, "every wave owns value tiles");
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::WALK_BYTES];
    bf16* const Qs = reinterpret_cast<bf16*>(smem);
    bf16* const Ks = Qs + Cf::K_OFF;
    bf16* const Vs = Qs + Cf::V_OFF;
    bf16* const Ps = Qs + Cf::P_OFF;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int NB = D / BV;  // value blocks per state
    const int64_t bh = blockIdx.x / NB;
    const int v0 = BV * (int)(blockIdx.x % NB);
    const int R = T * G;  // query rows
    const In* Qb = Q + bh * (int64_t)G * T * D;
    const In* Kb = K + bh * (int64_t)T * D;
    const In* Vb = V + bh * (int64_t)T * D;
    float* Ob = O + bh * (int64_t)G * T * D + v0;
    float* Sb = S + bh * (int64_t)D * D + v0;

    // S_0 straight into the accumulator layout (no column read when S_0 = 0)
    f32x4 Sacc[Cf::NVW][Cf::NDT];
    state_gmem_to_regs<Cf>(Sacc, Sb, D, D, zero_start ? 0 : BV, w, g, c16);
    // row r = t G + g of Q is token t of query head g
    stage_rows<In, D, Cf::LQ, 64, NTH>(Qs, R, [&](int r) { return Qb + ((int64_t)(r % G) * T + r / G) * D; }, tid);
    stage_rows<In, D, Cf::LK, 64, NTH>(Ks, T, [&](int r) { return Kb + (int64_t)r * D; }, tid);
    stage_rows<In, BV, Cf::LV, 64, NTH>(Vs, T, [&](int r) { return Vb + (int64_t)r * D + v0; }, tid);
    __syncthreads();

    const ScoreTiles<Cf> stiles(w);
    chunk_scores<Cf>(stiles, Qs, Ks, Ps, w, g, c16, NoHook(), G);
    __syncthreads();  // P complete

    Fr Vf[Cf::NVW][Cf::NTS];
    load_vfrags<Cf>(Vf, Vs, w, g, lane);
    f32x4 Oacc[Cf::NT][Cf::NVW];
    chunk_output<Cf>(Oacc, Sacc, Vf, Qs, Ps, w, g, c16);
    state_hop<Cf>(Sacc, Vf, Ks, w, g, lane);

    // Oacc[it][vw] holds O[row 16 it + c16][value columns 16 (w + NW vw) + 4g .. + 3]
#pragma unroll
    for (int it = 0; it < Cf::NT; ++it) {
        const int r = 16 * it + c16;
        if (r < R) {
            float* orow = Ob + ((int64_t)(r % G) * T + r / G) * D;
#pragma unroll
            for (int vw = 0; vw < Cf::NVW; ++vw)
                *reinterpret_cast<f32x4*>(orow + 16 * (w + NW * vw) + 4 * g) = Oacc[it][vw];
        }
    }
    state_regs_to_gmem<Cf>(Sb, Sacc, D, D, w, g, c16);
}

// The same continuation for d = 128, persistent and pipelined: one
// eight-wave workgroup (all 128 value columns, wave w owns value tile w)
// walks the key/value heads bh = blockIdx.x, blockIdx.x + gridDim.x, ...
// While head bh is computed, the loads of the next head -- its state rows and
// its Q, K and V rows, into registers -- are in flight.  The state moves
// between global memory and LDS as 16-byte row pieces (coalesced, like the
// decode step's), and between LDS and the accumulator layout inside the
// workgroup.  One workgroup per state reads its Q and K rows once.  The
// arithmetic per head is k_tokens_grouped's (the walk's chunk helpers), so
// the bits are the same.
constexpr int kGroupedPipeWGs = 256;  // workgroups of k_tokens_grouped_pipe (one per compute unit)

template <typename In>
__global__ __launch_bounds__(8 * kWave) void k_tokens_grouped_pipe(
    const In* __restrict__ Q, const In* __restrict__ K, const In* __restrict__ V, float* __restrict__ S,
    float* __restrict__ O, int64_t BHkv, int T, int G, int zero_start) {
    constexpr int D = 128, NW = 8;
    using Cf = WalkCfg<bf16, 64, D, D, NW>;
    using Fr = typename Cf::Fr;
    constexpr int NTH = Cf::NTH;
    static_assert(Cf::NVW == 1 && Cf::ALL_WAVES, "one value tile per wave");
    constexpr int KROWS = kDecodeTokensMax;     // key and value rows staged (T <= this)
    constexpr int SV = D * D / 4 / NTH;          // 16-byte state pieces per thread
    static_assert(SV * 4 * NTH == D * D, "the state splits evenly over the threads");
    // Q, K, V and P tiles, then the fp32 state (D rows of stride SLD)
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::WALK_BYTES + Cf::STATE_BYTES];
    bf16* const Qs = reinterpret_cast<bf16*>(smem);
    bf16* const Ks = Qs + Cf::K_OFF;
    bf16* const Vs = Qs + Cf::V_OFF;
    bf16* const Ps = Qs + Cf::P_OFF;
    float* const Sst = reinterpret_cast<float*>(smem + Cf::WALK_BYTES);

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int R = T * G;  // query rows, row r = t G + j is token t of query head j
    const int64_t q_elems = (int64_t)G * T * D;  // per key/value head
    const int64_t stride = gridDim.x;

    // Key and value rows past T stay zero for every head: rows KROWS.. are
    // cleared here, rows T..KROWS-1 are written as zeros by every scatter.
    for (int e = tid; e < (64 - KROWS) * D / 8; e += NTH) {
        const int row = KROWS + e / (D / 8), c8 = 8 * (e % (D / 8));
        *reinterpret_cast<u32x4*>(Ks + row * Cf::LK + c8) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(Vs + row * Cf::LV + c8) = u32x4{0u, 0u, 0u, 0u};
    }

    using TQ = Tile<bf16, 64, D, typename Cf::LQL, NTH, In>;
    using TK = Tile<bf16, KROWS, D, typename Cf::LKL, NTH, In>;
    using TV = Tile<bf16, KROWS, D, typename Cf::LVL, NTH, In>;
    TQ tq;
    TK tk;
    TV tv;
    tk.init(D, D, tid);
    tv.init(D, D, tid);
    u32x4 sp[SV];  // state piece n of this thread: row (tid + NTH n) / 32, columns 4 ((tid + NTH n) % 32) ..
    // The next head's rows into registers.  Q vector n of this thread: tile
    // row e / VPR, i.e. query row r, read from row (r % G) T + r / G of the
    // head's [G][T][D] block.
    auto gather = [&](int64_t bh) {
        const rsrc_t rq = make_rsrc(Q + bh * q_elems, (uint32_t)(q_elems * sizeof(In)));
#pragma unroll
        for (int n = 0; n < TQ::NPT; ++n) {
            const int e = tid + n * NTH, r = e / TQ::VPR, cv = e % TQ::VPR;
            const uint32_t off = r < R ? (uint32_t)((((r % G) * T + r / G) * D + cv * TQ::VE) * sizeof(In)) : kOutside;
            tq.r[n] = buf_load16(rq, off);
        }
        tk.gather(K + bh * (int64_t)T * D, D, T);
        tv.gather(V + bh * (int64_t)T * D, D, T);
        const rsrc_t rs = make_rsrc(S + bh * (int64_t)D * D, zero_start ? 0u : (uint32_t)(D * D * 4));
#pragma unroll
        for (int n = 0; n < SV; ++n) sp[n] = buf_load16(rs, (uint32_t)((tid + NTH * n) * 16));
    };

    const ScoreTiles<Cf> stiles(w);
    auto head = [&](int64_t bh) {
        const int64_t nx = bh + stride;
        __syncthreads();  // the previous head's readers of the tiles, P and the state area are done
        tq.scatter(Qs, tid);
        tk.scatter(Ks, tid);
        tv.scatter(Vs, tid);
#pragma unroll
        for (int n = 0; n < SV; ++n) {
            const int e = tid + NTH * n;
            *reinterpret_cast<u32x4*>(Sst + (e / (D / 4)) * Cf::SLD + 4 * (e % (D / 4))) = sp[n];
        }
        if (nx < BHkv) gather(nx);  // in flight during this head
        __syncthreads();

        f32x4 Sacc[1][Cf::NDT];
        state_lds_to_regs<Cf>(Sacc, Sst, w, g, c16);
        chunk_scores<Cf>(stiles, Qs, Ks, Ps, w, g, c16, NoHook(), G);
        __syncthreads();  // P complete; every wave has its state slice
        Fr Vf[1][Cf::NTS];
        load_vfrags<Cf>(Vf, Vs, w, g, lane);
        f32x4 Oacc[Cf::NT][1];
        chunk_output<Cf>(Oacc, Sacc, Vf, Qs, Ps, w, g, c16);
        state_hop<Cf>(Sacc, Vf, Ks, w, g, lane);

        // Oacc[it][0] holds O[row 16 it + c16][value columns 16 w + 4g .. + 3]
        const rsrc_t ro = make_rsrc(O + bh * q_elems, (uint32_t)(q_elems * 4));
#pragma unroll
        for (int it = 0; it < Cf::NT; ++it) {
            const int r = 16 * it + c16;
            const uint32_t off = r < R ? (uint32_t)((((r % G) * T + r / G) * D + 16 * w + 4 * g) * 4) : kOutside;
            buf_store16(ro, off, Oacc[it][0]);
        }
        state_regs_to_lds<Cf>(Sst, Sacc, w, g, c16);
        __syncthreads();
        const rsrc_t rs = make_rsrc(S + bh * (int64_t)D * D, (uint32_t)(D * D * 4));
#pragma unroll
        for (int n = 0; n < SV; ++n) {
            const int e = tid + NTH * n;
            buf_store16(rs, (uint32_t)(e * 16),
                        *reinterpret_cast<const f32x4*>(Sst + (e / (D / 4)) * Cf::SLD + 4 * (e % (D / 4))));
        }
    };
    // The first head outside the loop, so that the compiler's wait counts
    // for the prefetched registers need not merge the two ways they are
    // loaded (before the loop, and by the previous head).
    int64_t bh = blockIdx.x;
    if (bh >= BHkv) return;
    gather(bh);
    head(bh);
    for (bh += stride; bh < BHkv; bh += stride) head(bh);
}

// ---------------------------------------------------------------------------
// Phase 3, wide form for d = 128 bf16 (or FP8, staged as bf16) inputs:
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
    static constexpr int BYTES = (2 * BUF + Base::NP * Base::P_ELEMS) * 2;
};

// GATED: the gated walk (see k_gated_walk), the gates those of the key/value
// head; the chunk's decay prefix is double buffered (Bs2), written for chunk
// c + 1 by wave 0 while chunk c is computed.
template <int CT, typename In, bool GATED = false>
__global__ __launch_bounds__(kWideWaves * kWave) void k_chunk_walk_wide(
    const In* __restrict__ Q, const In* __restrict__ K, const In* __restrict__ V,
    float* __restrict__ S, float* __restrict__ O, const float* __restrict__ ws, int64_t T_len,
    int dk, int dv, int C, int64_t G, int64_t n_seg, int group, int zero_start, int keep,
    const float* __restrict__ gate) {
    using Cf = WideCfg<CT>;
    using Fr = typename Cf::Fr;
    constexpr int NTH = Cf::NTH;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::BYTES];
    __shared__ __attribute__((aligned(16))) float Bs2[GATED ? 2 : 1][GATED ? 3 * CT : 4];
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
    // gates of row r of chunk c (1 past the chunk's rows); wave 0 holds the
    // next chunk's in g0
    auto gate_of = [&](int64_t c, int r) { return r < rows_of(c) ? gate[bh * T_len + c * C + r] : 1.0f; };
    float g0 = 1.0f;
    if constexpr (GATED) {
        if (w == 0) {
            chunk_decay<CT>(Bs2[0], gate_of(c0, lane), lane);
            g0 = gate_of(c0 + 1, lane);
        }
    }

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
        const float* Bs = Bs2[GATED ? b : 0];
        auto out_hook = [&](int ds) {
            if (ds < Cf::NT) {
#pragma unroll
                for (int vw = 0; vw < Cf::NVW; ++vw) {
                    const int vcol = 16 * (w + Cf::NW * vw) + 4 * g;
                    const uint32_t off = vcol < dv ? (uint32_t)((c16 * dv + vcol) * 4) : kOutside;
                    buf_store16(rso, opaque(off) + (uint32_t)(16 * ds * dv * 4), Oacc[ds][vw]);
                }
            }
        };
        if constexpr (GATED)
            chunk_scores<Cf>(stiles, Qs, Ks, Ps, w, g, c16, out_hook, 0, DecayGate{Bs});
        else
            chunk_scores<Cf>(stiles, Qs, Ks, Ps, w, g, c16, out_hook);
        // The next chunk into the free buffer (its last readers finished
        // before the previous barrier).
        if (c + 1 < c1) {
            tq.scatter(nxt, tid);
            tk.scatter(nxt + Cf::K_OFF, tid);
            tv.scatter(nxt + Cf::V_OFF, tid);
            if constexpr (GATED)
                if (w == 0) chunk_decay<CT>(Bs2[1 - b], g0, lane);
        }
        __syncthreads();  // P complete
        if constexpr (GATED) {
            if (w == 0) {
                g0 = gate_of(c + 2, lane);
            }
        }

        const int64_t t2 = (c + 2) * C;
        const int n2 = rows_of(c + 2);
        const rsrc_t rq = tq.source(Qb + t2 * dk, dk, n2), rk = tk.source(Kb + t2 * dk, dk, n2),
                     rv = tv.source(Vb + t2 * dv, dv, n2);
        Fr Vf[Cf::NVW][Cf::NTS];
        load_vfrags<Cf>(Vf, Vs, w, g, lane);
        auto load_hook = [&](int ds) {
#pragma unroll
            for (int n = 0; n < decltype(tq)::NPT; ++n) {
                if (ds == 0) tq.load(rq, n);
                if (ds == 1) tk.load(rk, n);
                if (ds == 2) tv.load(rv, n);
            }
        };
        if constexpr (GATED)
            chunk_output<Cf>(Oacc, Sacc, Vf, Qs, Ps, w, g, c16, load_hook, DecayRows<CT>{Bs, c16});
        else
            chunk_output<Cf>(Oacc, Sacc, Vf, Qs, Ps, w, g, c16, load_hook);
        t_prev = c * C;
        n_prev = rows_of(c);
        if (c + 1 < c1 || (last_seg && !keep)) {
            if constexpr (GATED)
                state_hop_gated<Cf>(Sacc, Vf, Ks, Bs, w, g, lane);
            else
                state_hop<Cf>(Sacc, Vf, Ks, w, g, lane);
        }
        __syncthreads();  // this buffer and P free; the next buffer visible
    }
    store_out<Cf, true>(Ob, Oacc, t_prev, n_prev, dv, dv, w, g, c16);

    if (last_seg && bq % group == 0 && !keep)  // one writer per group; none for a verify pass
        state_regs_to_gmem<Cf>(S + bh * dkdv, Sacc, dk, dv, w, g, c16);
}

// ---------------------------------------------------------------------------
// Phase 1, wide form for d = 128 bf16 (or FP8) inputs:
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

// GATED: the gated segment pass (see k_gated_segment_states): the chunk's
// decay prefix double buffered like the tiles, the segment's total decay to
// dec[bh * n_seg + seg].
template <int CT, typename In, bool GATED = false>
__global__ __launch_bounds__(512) void k_segment_states_wide(const In* __restrict__ K,
                                                             const In* __restrict__ V,
                                                             float* __restrict__ ws, int64_t T_len,
                                                             int dk, int dv, int C, int64_t G,
                                                             int64_t n_seg, const float* __restrict__ gate,
                                                             float* __restrict__ dec) {
    using Cf = SegWideCfg<CT>;
    using Fr = typename Cf::Fr;
    constexpr int NTH = Cf::NTH;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::BYTES];
    __shared__ __attribute__((aligned(16))) float Bs2[GATED ? 2 : 1][GATED ? 3 * CT : 4];
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
    auto gate_of = [&](int64_t c, int r) { return r < rows_of(c) ? gate[bh * T_len + c * C + r] : 1.0f; };
    float g0 = 1.0f, L = 0.0f;
    if constexpr (GATED) {
        if (w == 0) {
            chunk_decay<CT>(Bs2[0], gate_of(c0, lane), lane);
            g0 = gate_of(c0 + 1, lane);
        }
    }
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
                if constexpr (GATED)
                    if (w == 0) chunk_decay<CT>(Bs2[1 - b], g0, lane);
            }
            // set u held chunk c, written to LDS one chunk ago: reload it
            const int64_t tn = (c + PF) * C;
            const int nn = rows_of(c + PF);
            const rsrc_t rk = tk[u].source(Kb + tn * dk, dk, nn), rv = tv[u].source(Vb + tn * dv, dv, nn);

            Fr Vf[Cf::NVW][Cf::NTS];
            load_vfrags<Cf>(Vf, Vs, w, g, lane);
            if constexpr (GATED) {
#pragma unroll
                for (int n = 0; n < TK::NPT; ++n) {
                    tk[u].load(rk, n);
                    tv[u].load(rv, n);
                }
                if (w == 0) {
                    g0 = gate_of(c + 2, lane);
                }
                state_hop_gated<Cf>(Sacc, Vf, Ks, Bs2[b], w, g, lane);
                L += Bs2[b][CT - 1];
            } else {
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
            }
            __syncthreads();  // this buffer free; the next one visible
        }
    }

    // (the loop ended with a barrier: the tiles are free)
    state_regs_to_lds<Cf>(Sst, Sacc, w, g, c16);
    __syncthreads();
    state_lds_to_gmem<Cf>(ws + (bh * n_seg + seg + 1) * (int64_t)dk * dv, Sst, dk, dv, dv, tid);
    if constexpr (GATED)
        if (tid == 0) dec[bh * n_seg + seg] = L;
}

// Gated phase 1: each segment's increment sum_t 2^{L_seg - b_t} k_t v_t^T
// (decays measured to the segment's end) into slot seg + 1, and its total
// decay L_seg (log2) into dec[bh * n_seg + seg].  One workgroup per (b,h),
// segment but the last, and value block.
template <typename In, int CT, int D, int BV, bool VEC>
__global__ __launch_bounds__(kThreads) void k_gated_segment_states(
    const In* __restrict__ K, const In* __restrict__ V, const float* __restrict__ gate,
    float* __restrict__ ws, float* __restrict__ dec, int64_t T_len, int dk, int dv, int C, int64_t G,
    int64_t n_seg, int n_vb) {
    using T = typename Compute<In>::type;
    using Cf = WalkCfg<T, CT, D, BV, kWaves>;
    using Fr = typename Cf::Fr;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::SEG_BYTES];
    __shared__ __attribute__((aligned(16))) float Bs[3 * CT];
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
    const float* gb = gate + bh * T_len;

    f32x4 Sacc[Cf::NVW][Cf::NDT];
#pragma unroll
    for (int vw = 0; vw < Cf::NVW; ++vw)
#pragma unroll
        for (int dt = 0; dt < Cf::NDT; ++dt) Sacc[vw][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto rows_of = [&](int64_t c) { return (int)min((int64_t)C, T_len - c * C); };
    auto gate_of = [&](int64_t c, int r) { return r < rows_of(c) ? gb[c * C + r] : 1.0f; };
    float L = 0.0f;  // the segment's decay so far (log2)

    using TK = Tile<T, CT, D, typename Cf::LKL, Cf::NTH, In>;
    using TV = Tile<T, CT, BV, typename Cf::LVL, Cf::NTH, In>;
    TK tk;
    TV tv;
    if constexpr (VEC) {
        tk.init(dk, dk, tid);
        tv.init(dv, nv, tid);
        tk.gather(Kb + c0 * C * dk, dk, rows_of(c0));
        tv.gather(Vb + c0 * C * dv, dv, rows_of(c0));
    }
    float g0 = 1.0f;
    if (w == 0) g0 = gate_of(c0, lane);
    for (int64_t c = c0; c < c1; ++c) {
        if constexpr (VEC) {
            tk.scatter(Ks, tid);
            tv.scatter(Vs, tid);
        } else {
            TK::load_scalar(Kb + c * C * dk, dk, rows_of(c), dk, Ks, tid);
            TV::load_scalar(Vb + c * C * dv, dv, rows_of(c), nv, Vs, tid);
        }
        if (w == 0) chunk_decay<CT>(Bs, g0, lane);
        __syncthreads();
        if (c + 1 < c1) {  // the next chunk's loads fly during this chunk's math
            if constexpr (VEC) {
                tk.gather(Kb + (c + 1) * C * dk, dk, rows_of(c + 1));
                tv.gather(Vb + (c + 1) * C * dv, dv, rows_of(c + 1));
            }
            if (w == 0) {
                g0 = gate_of(c + 1, lane);
            }
        }
        Fr Vf[Cf::NVW][Cf::NTS];
        load_vfrags<Cf>(Vf, Vs, w, g, lane);
        state_hop_gated<Cf>(Sacc, Vf, Ks, Bs, w, g, lane);
        L += Bs[CT - 1];
        __syncthreads();
    }
    // (the loop ended with a barrier: the tiles are free)
    state_regs_to_lds<Cf>(Sst, Sacc, w, g, c16);
    __syncthreads();
    state_lds_to_gmem<Cf>(ws + (bh * n_seg + seg + 1) * (int64_t)dk * dv + v0, Sst, dk, dv, nv, tid);
    if (vb == 0 && tid == 0) dec[bh * n_seg + seg] = L;
}

// Gated phase 2: slot 0 = S_0, slot s = 2^{L_{s-1}} slot (s-1) + increment
// (s - 1).  Four consecutive state elements of one (b,h) per thread.
__global__ __launch_bounds__(kThreads) void k_gated_state_scan(const float* __restrict__ S,
                                                               float* __restrict__ ws,
                                                               const float* __restrict__ dec,
                                                               int64_t n_seg, int64_t dkdv,
                                                               int64_t blocks_per_bh, int zero_start) {
    const int64_t bh = blockIdx.x / blocks_per_bh;
    const int64_t e = ((blockIdx.x % blocks_per_bh) * kThreads + threadIdx.x) * 4;
    if (e >= dkdv) return;
    float* slot = ws + bh * n_seg * dkdv + e;
    const float* L = dec + bh * n_seg;
    const float* s0 = S + bh * dkdv + e;
    if (e + 4 <= dkdv && (dkdv & 3) == 0) {
        // as k_state_scan: slot 0 and the first U increments loaded together,
        // then folded in segment order (slot 0 is written even for a single
        // segment: grouped heads read their start state there)
        constexpr int U = 16;
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
                    const float f = exp2f(L[s + u - 1]);  // the previous segment's total decay
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] = fmaf(f, acc[r], x[u][r]);
                    *reinterpret_cast<f32x4*>(slot + (s + u) * dkdv) = acc;
                }
        }
    } else {
        const int m = (int)min((int64_t)4, dkdv - e);
        for (int j = 0; j < m; ++j) {
            float acc = zero_start ? 0.0f : s0[j];
            slot[j] = acc;
            for (int64_t s = 1; s < n_seg; ++s) {
                acc = fmaf(exp2f(L[s - 1]), acc, slot[s * dkdv + j]);
                slot[s * dkdv + j] = acc;
            }
        }
    }
}

// Gated phase 3: the chunk walk of k_chunk_walk with the decays (one query
// head per state).
template <typename In, int CT, int D, int BV, bool VEC>
__global__ __launch_bounds__(kThreads) void k_gated_walk(
    const In* __restrict__ Q, const In* __restrict__ K, const In* __restrict__ V,
    const float* __restrict__ gate, float* __restrict__ S, float* __restrict__ O,
    const float* __restrict__ ws, int64_t T_len, int dk, int dv, int C, int64_t G, int64_t n_seg,
    int n_vb, int group, int zero_start, int keep) {
    using T = typename Compute<In>::type;
    using Cf = WalkCfg<T, CT, D, BV, kWaves>;
    using Fr = typename Cf::Fr;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::WALK_BYTES];
    __shared__ __attribute__((aligned(16))) float Bs[3 * CT];
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
    // key/value head bh = bq / group: its K, V, gates and states
    const int64_t bq = line / n_seg, seg = line - bq * n_seg, bh = bq / group;
    const ScoreTiles<Cf> stiles(w);
    const int v0 = vb * BV;
    const int nv = min(BV, dv - v0);
    const int64_t n_c = (T_len + C - 1) / C;
    const int64_t c0 = seg * G, c1 = min(n_c, c0 + G);
    const bool last_seg = seg == n_seg - 1;
    const int64_t dkdv = (int64_t)dk * dv;
    const In* Qb = Q + bq * T_len * dk;
    const In* Kb = K + bh * T_len * dk;
    const In* Vb = V + bh * T_len * dv + v0;
    const float* gb = gate + bh * T_len;
    float* Ob = O + bq * T_len * dv + v0;

    // Incoming state of this segment, columns [v0, v0 + nv) (zero_start
    // without a workspace: S_0 = 0, S is not read)
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
    auto gate_of = [&](int64_t c, int r) { return r < rows_of(c) ? gb[c * C + r] : 1.0f; };
    if constexpr (VEC) {
        tq.init(dk, dk, tid);
        tk.init(dk, dk, tid);
        tv.init(dv, nv, tid);
        tq.gather(Qb + c0 * C * dk, dk, rows_of(c0));
        tk.gather(Kb + c0 * C * dk, dk, rows_of(c0));
        tv.gather(Vb + c0 * C * dv, dv, rows_of(c0));
    }
    float g0 = 1.0f;
    if (w == 0) g0 = gate_of(c0, lane);

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
        if (w == 0) chunk_decay<CT>(Bs, g0, lane);
        __syncthreads();
        if (c > c0) store_out<Cf, VEC>(Ob, Oacc, t_prev, n_prev, nv, dv, w, g, c16);
        if (c + 1 < c1) {  // the next chunk's loads fly during this chunk's math
            if constexpr (VEC) {
                const int nr = rows_of(c + 1);
                tq.gather(Qb + (t0 + C) * dk, dk, nr);
                tk.gather(Kb + (t0 + C) * dk, dk, nr);
                tv.gather(Vb + (t0 + C) * dv, dv, nr);
            }
            if (w == 0) {
                g0 = gate_of(c + 1, lane);
            }
        }

        chunk_scores<Cf>(stiles, Qs, Ks, Ps, w, g, c16, NoHook(), 0, DecayGate{Bs});
        __syncthreads();
        Fr Vf[Cf::NVW][Cf::NTS];
        load_vfrags<Cf>(Vf, Vs, w, g, lane);
        chunk_output<Cf>(Oacc, Sacc, Vf, Qs, Ps, w, g, c16, NoHook(), DecayRows<CT>{Bs, c16});
        t_prev = t0;
        n_prev = nrows;
        if (c + 1 < c1 || (last_seg && !keep)) state_hop_gated<Cf>(Sacc, Vf, Ks, Bs, w, g, lane);
        __syncthreads();
    }
    if (c1 > c0) store_out<Cf, VEC>(Ob, Oacc, t_prev, n_prev, nv, dv, w, g, c16);

    // S_T: one writer per group (the loop ended with a barrier); none for a
    // verify pass, which leaves S as it was
    if (last_seg && !keep && bq % group == 0) {
        state_regs_to_lds<Cf>(Sst, Sacc, w, g, c16);
        __syncthreads();
        state_lds_to_gmem<Cf>(S + bh * dkdv + v0, Sst, dk, dv, nv, tid);
    }
}

// ---------------------------------------------------------------------------
// Host side: dispatch over (input type, chunk tile, head dim); the plan
// itself is made in lla_plan.cpp.
// ---------------------------------------------------------------------------
// In: the input element type (bf16, FP8 or fp32); the matrix cores run on
// Compute<In>::type.
template <typename In, int CT, int D>
static hipError_t launch_walk_t(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                                float* S, float* O, float* ws, hipStream_t st) {
    using T = typename Compute<In>::type;
    if constexpr (std::is_same<T, bf16>::value && D == 128) {
        if (p.vec) {  // one eight-wave workgroup per (b,h) and segment
            hipLaunchKernelGGL((k_chunk_walk_wide<CT, In>), dim3((unsigned)(p.BHq * p.n_seg)), dim3(kWideWaves * kWave), 0, st,
                               (const In*)Q, (const In*)K, (const In*)V, S, O,
                               (const float*)(p.use_ws ? ws : nullptr), p.T, p.dk, p.dv, p.C, p.G,
                               p.n_seg, p.group, (int)p.zero_start, (int)p.keep, (const float*)nullptr);
            return hipGetLastError();
        }
    }
    constexpr int BV = D > 64 ? 64 : D;
    const int64_t grid = p.BHq * p.n_seg * p.n_vb;
    const float* wsr = p.use_ws ? ws : nullptr;
    if constexpr (!std::is_same<In, float>::value) {  // (fp32 inputs keep the three phases)
        if (p.prefix) {  // each walk sums the segments before its own, or reads their published sums
            float* pub = p.publish ? ws : nullptr;
            unsigned long long* fl =
                p.publish ? reinterpret_cast<unsigned long long*>(ws + prefix_slot_floats(p)) : nullptr;
            if (p.vec)
                hipLaunchKernelGGL((k_chunk_walk<In, CT, D, BV, true, kWaves, true>), dim3((unsigned)grid),
                                   dim3(kThreads), 0, st, (const In*)Q, (const In*)K, (const In*)V, S, O,
                                   (const float*)nullptr, p.T, p.dk, p.dv, p.C, p.G, p.n_seg, p.n_vb, p.group,
                                   (int)p.zero_start, (int)p.keep, pub, fl, p.token, p.wait_ticks);
            else
                hipLaunchKernelGGL((k_chunk_walk<In, CT, D, BV, false, kWaves, true>), dim3((unsigned)grid),
                                   dim3(kThreads), 0, st, (const In*)Q, (const In*)K, (const In*)V, S, O,
                                   (const float*)nullptr, p.T, p.dk, p.dv, p.C, p.G, p.n_seg, p.n_vb, p.group,
                                   (int)p.zero_start, (int)p.keep, pub, fl, p.token, p.wait_ticks);
            return hipGetLastError();
        }
    }
    if (p.vec)
        hipLaunchKernelGGL((k_chunk_walk<In, CT, D, BV, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                           st, (const In*)Q, (const In*)K, (const In*)V, S, O, wsr, p.T,
                           p.dk, p.dv, p.C, p.G, p.n_seg, p.n_vb, p.group, (int)p.zero_start, (int)p.keep,
                           (float*)nullptr, (unsigned long long*)nullptr, 0ull, (uint64_t)0);
    else
        hipLaunchKernelGGL((k_chunk_walk<In, CT, D, BV, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                           st, (const In*)Q, (const In*)K, (const In*)V, S, O, wsr, p.T,
                           p.dk, p.dv, p.C, p.G, p.n_seg, p.n_vb, p.group, (int)p.zero_start, (int)p.keep,
                           (float*)nullptr, (unsigned long long*)nullptr, 0ull, (uint64_t)0);
    return hipGetLastError();
}

template <typename In, int CT, int D>
static hipError_t launch_seg_t(const PrefillPlan& p, const void* K, const void* V, float* ws,
                               hipStream_t st) {
    using T = typename Compute<In>::type;
    if constexpr (std::is_same<T, bf16>::value && D == 128) {
        if (p.vec) {  // one eight-wave workgroup per (b,h) and segment
            hipLaunchKernelGGL((k_segment_states_wide<CT, In>), dim3((unsigned)(p.BH * (p.n_seg - 1))),
                               dim3(512), 0, st, (const In*)K, (const In*)V, ws, p.T, p.dk, p.dv,
                               p.C, p.G, p.n_seg, (const float*)nullptr, (float*)nullptr);
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
            } else {                                                                       \
                if (p.D == 32) return FN<fp8e4m3, 64, 32>(__VA_ARGS__);                    \
                if (p.D == 64) return FN<fp8e4m3, 64, 64>(__VA_ARGS__);                    \
                return FN<fp8e4m3, 64, 128>(__VA_ARGS__);                                  \
            }                                                                              \
        } else if (p.dtype == LLA_BF16) {                                                  \
            if (p.CT == 32) {                                                              \
                if (p.D == 32) return FN<bf16, 32, 32>(__VA_ARGS__);                       \
                if (p.D == 64) return FN<bf16, 32, 64>(__VA_ARGS__);                       \
                return FN<bf16, 32, 128>(__VA_ARGS__);                                     \
            } else {                                                                       \
                if (p.D == 32) return FN<bf16, 64, 32>(__VA_ARGS__);                       \
                if (p.D == 64) return FN<bf16, 64, 64>(__VA_ARGS__);                       \
                return FN<bf16, 64, 128>(__VA_ARGS__);                                     \
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


template <typename In>
static hipError_t tokens_grouped_t(const void* q, const void* k, const void* v, int64_t BHkv, int T, int G,
                                   int d, float* S, float* o, int zero, hipStream_t st) {
    if (d == 128) {
        const int64_t wgs = BHkv < kGroupedPipeWGs ? BHkv : kGroupedPipeWGs;
        hipLaunchKernelGGL((k_tokens_grouped_pipe<In>), dim3((unsigned)wgs), dim3(8 * kWave), 0, st, (const In*)q,
                           (const In*)k, (const In*)v, S, o, BHkv, T, G, zero);
    } else {
        hipLaunchKernelGGL((k_tokens_grouped<In, 64, 64, 4>), dim3((unsigned)BHkv), dim3(4 * kWave), 0, st,
                           (const In*)q, (const In*)k, (const In*)v, S, o, T, G, zero);
    }
    return hipGetLastError();
}

hipError_t launch_tokens_grouped(lla_dtype dtype, const void* q, const void* k, const void* v, int64_t BHkv,
                                 int T, int group, int d, float* S, float* o, bool zero_start, hipStream_t st) {
    const int z = zero_start ? 1 : 0;
    if (dtype == LLA_FP8_E4M3) return tokens_grouped_t<fp8e4m3>(q, k, v, BHkv, T, group, d, S, o, z, st);
    return tokens_grouped_t<bf16>(q, k, v, BHkv, T, group, d, S, o, z, st);
}

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

// ---- the gated walk: the four-wave kernels for every shape ---------------------

template <typename In, int CT, int D>
static hipError_t launch_gated_seg_t(const PrefillPlan& p, const void* K, const void* V, const float* gate,
                                     float* ws, float* dec, hipStream_t st) {
    using T = typename Compute<In>::type;
    if constexpr (std::is_same<T, bf16>::value && D == 128) {
        if (p.vec) {  // one eight-wave workgroup per (b,h) and segment
            hipLaunchKernelGGL((k_segment_states_wide<CT, In, true>), dim3((unsigned)(p.BH * (p.n_seg - 1))),
                               dim3(512), 0, st, (const In*)K, (const In*)V, ws, p.T, p.dk, p.dv, p.C, p.G,
                               p.n_seg, gate, dec);
            return hipGetLastError();
        }
    }
    constexpr int BV = D > 64 ? 64 : D;
    const int64_t grid = p.BH * (p.n_seg - 1) * p.n_vb;
    if (p.vec)
        hipLaunchKernelGGL((k_gated_segment_states<In, CT, D, BV, true>), dim3((unsigned)grid), dim3(kThreads),
                           0, st, (const In*)K, (const In*)V, gate, ws, dec, p.T, p.dk, p.dv, p.C, p.G, p.n_seg,
                           p.n_vb);
    else
        hipLaunchKernelGGL((k_gated_segment_states<In, CT, D, BV, false>), dim3((unsigned)grid), dim3(kThreads),
                           0, st, (const In*)K, (const In*)V, gate, ws, dec, p.T, p.dk, p.dv, p.C, p.G, p.n_seg,
                           p.n_vb);
    return hipGetLastError();
}

template <typename In, int CT, int D>
static hipError_t launch_gated_walk_t(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                                      const float* gate, float* S, float* O, float* ws, hipStream_t st) {
    using T = typename Compute<In>::type;
    if constexpr (std::is_same<T, bf16>::value && D == 128) {
        if (p.vec) {  // one eight-wave workgroup per (b,h) and segment
            hipLaunchKernelGGL((k_chunk_walk_wide<CT, In, true>), dim3((unsigned)(p.BHq * p.n_seg)),
                               dim3(kWideWaves * kWave), 0, st, (const In*)Q, (const In*)K, (const In*)V, S, O,
                               (const float*)(p.use_ws ? ws : nullptr), p.T, p.dk, p.dv, p.C, p.G, p.n_seg,
                               p.group, (int)p.zero_start, (int)p.keep, gate);
            return hipGetLastError();
        }
    }
    constexpr int BV = D > 64 ? 64 : D;
    const int64_t grid = p.BHq * p.n_seg * p.n_vb;
    const float* wsr = p.use_ws ? ws : nullptr;
    if (p.vec)
        hipLaunchKernelGGL((k_gated_walk<In, CT, D, BV, true>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                           (const In*)Q, (const In*)K, (const In*)V, gate, S, O, wsr, p.T, p.dk, p.dv, p.C, p.G,
                           p.n_seg, p.n_vb, p.group, (int)p.zero_start, (int)p.keep);
    else
        hipLaunchKernelGGL((k_gated_walk<In, CT, D, BV, false>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                           (const In*)Q, (const In*)K, (const In*)V, gate, S, O, wsr, p.T, p.dk, p.dv, p.C, p.G,
                           p.n_seg, p.n_vb, p.group, (int)p.zero_start, (int)p.keep);
    return hipGetLastError();
}

hipError_t launch_gated_prefill(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                                const float* gate, float* S, float* O, float* ws, hipStream_t st) {
    if (p.n_c == 0) return hipSuccess;
    if (p.use_ws) {  // several segments, or several query heads per state (slot 0 = S_0)
        const int64_t dkdv = (int64_t)p.dk * p.dv;
        float* dec = ws + p.BH * p.n_seg * dkdv;  // after the states
        hipError_t e = hipSuccess;
        if (p.n_seg > 1) e = [&]() -> hipError_t { LLA_DISPATCH(launch_gated_seg_t, p, K, V, gate, ws, dec, st); }();
        if (e != hipSuccess) return e;
        const int64_t per_block = (int64_t)kThreads * 4;  // four elements per thread
        const int64_t blocks_per_bh = (dkdv + per_block - 1) / per_block;
        hipLaunchKernelGGL(k_gated_state_scan, dim3((unsigned)(p.BH * blocks_per_bh)), dim3(kThreads), 0, st, S,
                           ws, dec, p.n_seg, dkdv, blocks_per_bh, (int)p.zero_start);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    LLA_DISPATCH(launch_gated_walk_t, p, Q, K, V, gate, S, O, ws, st);
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
