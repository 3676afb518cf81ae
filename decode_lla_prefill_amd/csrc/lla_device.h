// lla_device.h -- device-side building blocks shared by the HIP kernels of
// liblla (gfx950 only): vector types, the 16x16 matrix-core step, bf16
// rounding, FP8 (E4M3) decoding, and global->LDS tile staging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // four waves per workgroup
constexpr int kWaves = kThreads / kWave;

// x, hidden from the optimiser: arithmetic on the result is redone where it
// is used instead of being hoisted out of a loop into registers that stay
// live across it (an empty asm statement that claims to modify x; no
// instruction is emitted).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// One 32-deep slice of a 16x16 matrix-core product, held 8 elements per lane.
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

// c += a * b for a 16x32 by 32x16 slice.  Lane l supplies row (of a) or
// column (of b) l % 16 and eight depth slots; slot i of lane l pairs with
// slot i of the lanes of the same group l / 16.  Any assignment of depth
// indices to (group, slot) works as long as a and b use the same one.
// Result layout: lane l holds rows 4*(l/16) + {0,1,2,3} of column l % 16.
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
}

// FP8 inputs: the OCP 8-bit float with 4 exponent bits (bias 7) and 3
// mantissa bits, subnormals, no infinities, NaN = S.1111.111 -- the format
// torch calls float8_e4m3fn.  Every such value is a bf16 value, so decoding
// is exact; gfx950's conversion instructions decode this format (checked on
// all 256 codes against the format's definition).
struct fp8e4m3 {
    uint8_t bits;
};
static_assert(sizeof(fp8e4m3) == 1, "one byte per element");

// Four FP8 values (byte i of w = element i) -> bf16 pairs {e0, e1}, {e2, e3}.
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// The type the matrix cores take for a given input type: FP8 inputs are
// staged as bf16.
template <typename In> struct Compute { typedef In type; };
template <> struct Compute<fp8e4m3> { typedef bf16 type; };

// A decay gate as the kernels take it: g in [2^-126, 1] (g <= 0 and NaN act
// as 2^-126, g > 1 as 1).  The gated prefill works with log2 of it, clamped
// to the same range.
__device__ __forceinline__ float decay_gate(float g) { return fminf(fmaxf(g, 0x1p-126f), 1.0f); }

__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }  // round to nearest even
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(fp8e4m3 x) {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.bits, false);  // element 0 = byte 0
    return f[0];
}
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Input element -> the staged type (exact for every pair used here).
template <typename T> __device__ __forceinline__ T stage(T x) { return x; }
template <typename T> __device__ __forceinline__ T stage(fp8e4m3 x) { return from_f32<T>(to_f32(x)); }

// Elements per 16-byte vector.
template <typename T> struct Vec { static constexpr int n = 16 / sizeof(T); };

// ---- LDS tile layouts: (row, col) -> element offset ---------------------------

// Plain row-major tile with LD elements per row (LD a multiple of 4).
template <int LD>
struct PadLayout {
    static constexpr int kRowElems = LD;
    __device__ __forceinline__ static int off(int row, int col) { return row * LD + col; }
};

// ---- buffer (descriptor-based) global access ----------------------------------
//
// A buffer descriptor covers [base, base + bytes); a load whose offset falls
// outside returns zero and a store outside is dropped.  Tiles therefore need
// no per-lane branches: padding rows and columns get an offset past the end.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutside = 0x80000000u;  // an offset beyond every descriptor here
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // dword 3 = 0x00020000: raw (untyped) 32-bit data, the gfx9-family setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// The whole offset goes in the lane's offset operand (the scalar offset is
// left at zero), so the range check covers all of it.
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

// A ROWS x COLS tile of T staged in LDS with layout L, read from global
// memory holding elements of type In (T itself, or FP8 decoded to bf16 on
// the way into LDS).
//
// Staging is split in two halves so that the global loads of the next tile
// can be in flight while the current one is being used: gather() issues the
// 16-byte loads into registers, scatter() writes them to LDS.  Rows at or past
// `nrows`, and columns at or past `ncols`, are stored as zero.
template <typename T, int ROWS, int COLS, typename L, int NTH = kThreads, typename In = T>
struct Tile {
    static constexpr int VE = Vec<In>::n;           // elements per 16-byte global vector
    static constexpr int VPR = COLS / VE;           // vectors per row
    static constexpr int NV = ROWS * VPR;           // vectors per tile
    static constexpr int NPT = (NV + NTH - 1) / NTH;  // per thread (NTH threads)
    static constexpr bool FULL = NV % NTH == 0;
    static_assert(COLS % VE == 0, "tile width must be a whole number of vectors");
    static_assert(NTH % VPR == 0, "a thread's vectors share one column");

    u32x4 r[NPT];
    // Vector n of this thread is (row tid / VPR + n * NTH / VPR, column
    // vector tid % VPR): byte offset off + n * step within a tile (computed
    // next to each load, so one register holds all of them).  `off` is
    // kOutside for a padding column (kOutside + n * step stays outside:
    // n * step < 2^31); rows at or past the tile's last valid row, vectors
    // past the tile included, fall outside the descriptor.
    uint32_t off;
    uint32_t step;  // the same for every thread

    // Vector path set-up: global row stride `ld` elements (a multiple of VE),
    // valid columns `ncols` (a multiple of VE).  Offsets are the same for
    // every tile of a sequence.
    __device__ __forceinline__ void init(int64_t ld, int ncols, int tid) {
        const int row = tid / VPR, cv = tid % VPR;
        off = cv * VE < ncols ? (uint32_t)((row * ld + cv * VE) * sizeof(In)) : kOutside;
        step = (uint32_t)((NTH / VPR) * ld * sizeof(In));
    }
    // Loads the tile whose first row is at g; rows >= nrows read as zero.
    __device__ __forceinline__ void gather(const In* __restrict__ g, int64_t ld, int nrows) {
        const rsrc_t rs = source(g, ld, nrows);
#pragma unroll
        for (int n = 0; n < NPT; ++n) load(rs, n);
    }
    // The same in parts: the descriptor of a tile, then its n-th load.
    __device__ __forceinline__ static rsrc_t source(const In* __restrict__ g, int64_t ld, int nrows) {
        return make_rsrc(g, (uint32_t)(nrows * ld * sizeof(In)));
    }
    __device__ __forceinline__ void load(rsrc_t rs, int n) { r[n] = buf_load16(rs, opaque(off) + n * step); }
    __device__ __forceinline__ void scatter(T* lds, int tid) const {
#pragma unroll
        for (int n = 0; n < NPT; ++n) {
            const int e = tid + n * NTH;
            if (FULL || e < NV) {
                const int row = e / VPR, cv = e % VPR;
                if constexpr (sizeof(In) == sizeof(T)) {
                    *reinterpret_cast<u32x4*>(lds + L::off(row, cv * VE)) = r[n];
                } else {  // 16 FP8 values -> two 8-element bf16 vectors
                    static_assert(sizeof(In) == 1 && sizeof(T) == 2, "FP8 stages as bf16");
                    uint32_t x[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) fp8x4_to_bf16(r[n][i], x[2 * i], x[2 * i + 1]);
                    *reinterpret_cast<u32x4*>(lds + L::off(row, cv * VE)) = u32x4{x[0], x[1], x[2], x[3]};
                    *reinterpret_cast<u32x4*>(lds + L::off(row, cv * VE + 8)) = u32x4{x[4], x[5], x[6], x[7]};
                }
            }
        }
    }
    // Element path for shapes the vector path cannot take: straight to LDS.
    __device__ __forceinline__ static void load_scalar(const In* __restrict__ g, int64_t ld,
                                                       int nrows, int ncols, T* lds, int tid) {
        for (int e = tid; e < ROWS * COLS; e += NTH) {
            const int row = e / COLS, col = e % COLS;
            T x = from_f32<T>(0.0f);
            if (row < nrows && col < ncols) x = stage<T>(g[(int64_t)row * ld + col]);
            lds[L::off(row, col)] = x;
        }
    }
};

}  // namespace lla
