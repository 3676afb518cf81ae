// lla_internal.h -- host-side contract between the C ABI (lla_abi.cpp) and
// the kernel launchers (lla_prefill.hip, lla_decode.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lla.h"

namespace lla {

// Workgroups the chunk walk aims to launch: two per compute unit of a
// 256-CU MI355X.  A constant (not a device query) so that the segmentation,
// and therefore the rounding order, depends on the shape alone.
#ifndef LLA_TARGET_WALKERS
#define LLA_TARGET_WALKERS 512
#endif
constexpr int64_t kTargetWalkers = LLA_TARGET_WALKERS;

// Chunks of up to 64 tokens carry the masked scores P into P V as a bf16
// high + low pair (1), not as one bf16 value (0).
#ifndef LLA_SPLIT_P
#define LLA_SPLIT_P 1
#endif

// Everything the launchers need about a prefill shape, derived once on the
// host from the user's sizes.
struct PrefillPlan {
    int64_t B, H, BH, T;  // H: query heads; BH = B * Hkv (key/value heads, states)
    int64_t Hkv;          // key/value heads (0 on input: H)
    int group;            // query heads per key/value head = H / Hkv
    int64_t BHq;          // B * H
    bool use_ws;          // the walk starts every segment from the workspace
    int dk, dv, C;
    int D;        // padded head dim (32, 64 or 128) used for both dk and dv
    int CT;       // padded chunk tile (32, 64 or 128 rows)
    int BV;       // value columns per workgroup (D, or 64 when D = 128)
    int n_vb;     // value-column blocks = D / BV
    int64_t n_c;  // chunks per sequence = ceil(T / C)
    int64_t G;    // chunks per segment (walked by one workgroup)
    int64_t n_seg;  // segments per sequence = ceil(n_c / G)
    bool vec;     // 16-byte vector loads possible (dk, dv multiples of one vector)
    bool zero_start;  // S_0 = 0: S is written (S_T) but not read
    lla_dtype dtype;
};

// Fills the derived fields from B, H, T, dk, dv, C, dtype (already validated).
void plan_prefill(PrefillPlan& p);

hipError_t launch_segment_states(const PrefillPlan& p, const void* K, const void* V,
                                 float* ws, hipStream_t st);
hipError_t launch_state_scan(const PrefillPlan& p, const float* S, float* ws, hipStream_t st);
hipError_t launch_chunk_walk(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                             float* S, float* O, float* ws, hipStream_t st);

hipError_t launch_decode_step(lla_dtype dtype, const void* q, const void* k, const void* v,
                              int64_t BH, int dk, int dv, float* S, float* o, hipStream_t st);

// Short prompts (T <= kDecodeTokensMax tokens, dk = dv in {64, 128}; with
// shared-state heads, T * group <= kDecodeTokensQueries) run as T fused decode
// steps with the state in registers; lla_prefill takes this route when
// decode_tokens_fit() holds.  One workgroup per key/value head.
constexpr int kDecodeTokensMax = 16;
constexpr int kDecodeTokensQueries = 64;
bool decode_tokens_fit(int64_t T, int dk, int dv, int64_t group);
hipError_t launch_decode_tokens(lla_dtype dtype, const void* q, const void* k, const void* v,
                                int64_t BHkv, int T, int group, int d, float* S, float* o,
                                bool zero_start, hipStream_t st);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

// Shared-state heads: `group` query heads read each key/value state (dk = dv
// in {64, 128}, group <= kDecodeGroupMax).  q, o: [BHkv * group][d].
constexpr int kDecodeGroupMax = 16;
bool decode_group_fit(int64_t group, int dk, int dv);
hipError_t launch_decode_group(lla_dtype dtype, const void* q, const void* k, const void* v,
                               int64_t BHkv, int group, int d, float* S, float* o, hipStream_t st);

}  // namespace lla
