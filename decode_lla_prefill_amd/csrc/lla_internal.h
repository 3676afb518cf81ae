// lla_internal.h -- host-side contract between the C ABI (lla_abi.cpp) and
// the kernel launchers (lla_prefill.hip, lla_decode.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lla.h"

namespace lla {

// (sequence, head, segment) lines the chunk walk aims for: one per compute
// unit of a 256-CU MI355X.  A line is one eight-wave workgroup (d = 128,
// bf16 or FP8), or one four-wave workgroup per block of value columns.
// Measured: at T = 8192 (d = 128) fewer, longer lines lose parallelism; at
// T = 1024 (d = 64) one line per CU (two chunks each) beats two (one chunk
// each: the segment pass, the scan and the walk are then all fixed cost).
// A constant (not a device query) so that the segmentation, and therefore
// the rounding order, depends on the shape alone.
#ifndef LLA_TARGET_WALKERS
#define LLA_TARGET_WALKERS 256
#endif
constexpr int64_t kTargetWalkers = LLA_TARGET_WALKERS;

// The masked scores P enter P V as a bf16 high + low pair (1), not as one
// bf16 value (0).
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
    int dk, dv, C;  // C: the chunk run (the caller's, or half of one over 64 tokens)
    int D;        // padded head dim (32, 64 or 128) used for both dk and dv
    int CT;       // padded chunk tile (32 or 64 rows; C > 64 runs as two sub-chunks)
    int BV;       // value columns per workgroup (D, or 64 when D = 128)
    int n_vb;     // value-column blocks = D / BV
    int64_t n_c;  // chunks per sequence = ceil(T / C)
    int64_t G;    // chunks per segment (walked by one workgroup)
    int64_t n_seg;  // segments per sequence = ceil(n_c / G)
    bool vec;     // 16-byte vector loads possible (dk, dv multiples of one vector)
    bool zero_start;  // S_0 = 0: S is written (S_T) but not read
    bool keep;        // the verify pass: S is read (unless zero_start) but never written
    bool prefix;      // one launch: every walk sums the segments before its own (prefix_walk_fits)
    bool publish;     // ... and reads the earlier segments' sums from the workspace where published
    unsigned long long token;  // this call's flag value for the published sums (never 0)
    uint64_t wait_ticks;       // a reader's wait for them (100 MHz ticks; lla_set_publish_wait_ticks)
    lla_dtype dtype;
};

// Fills the derived fields from B, H, T, dk, dv, C, dtype (already validated).
void plan_prefill(PrefillPlan& p);

// Whether lla_prefill runs as one walk whose workgroups sum the earlier
// segments' K^T V themselves (same bits as the three phases): bf16 or FP8
// inputs on the four-wave walk, several segments, S not both read and
// written (a fresh prompt or a verify pass), and at most kPrefixMaxChunks
// chunks before the last segment.  Measured: at 12-15 chunks before the
// last segment the one launch is 0-16 % faster than the three phases (2-4 µs
// saved on 10-25 µs steps), at 28-60 chunks 20-90 % slower; fp32 inputs,
// whose state hop costs more, were slower at 14.  Needs zero_start and
// keep set.
#ifndef LLA_PREFIX_MAX_CHUNKS
#define LLA_PREFIX_MAX_CHUNKS 16
#endif
constexpr int64_t kPrefixMaxChunks = LLA_PREFIX_MAX_CHUNKS;
// With the earlier segments' sums published (see below): at most 16 segments,
// 8 chunks per segment (a writer's own sum stays well inside the readers'
// bounded wait) and 64 chunks before the last one.  Measured (fresh prompts,
// d = 64 and 32, T = 2048-4096, G = 2-8): up to 15 % faster than the three
// phases with cold inputs at 8-16 segments, 17 % slower at 32; without
// publication such shapes keep the three phases (summing 28-60 chunks again
// measured 20-90 % slower).
constexpr int64_t kPublishMaxSegments = 16;
constexpr int64_t kPublishMaxChunks = 64;
constexpr int64_t kPublishMaxG = 8;
// How long a walk waits for an earlier segment's published sum before it sums
// that segment itself, by default: 2,000 ticks of the 100 MHz real-time
// counter (20 us; a writer's own sum takes a few).
constexpr uint64_t kPublishWaitTicks = 2000;
// `published`: the call can publish (workspace large enough, stream not
// capturing), which admits the larger shapes above.
bool prefix_walk_fits(const PrefillPlan& p, bool published);

// The one-launch walk's published segment sums (the kernel's layout): one
// slot of 64 * D floats per (key/value head, segment, value block) -- four
// waves, one value tile each, D / 16 key tiles of 16 x 16 -- then one 8-byte
// flag per slot.  prefix_capable: the shape could take the one-launch walk
// for some dtype and options, so the workspace size covers the slots.
bool prefix_capable(const PrefillPlan& p);
int64_t prefix_slot_floats(const PrefillPlan& p);
size_t prefix_publish_bytes(const PrefillPlan& p);

hipError_t launch_segment_states(const PrefillPlan& p, const void* K, const void* V,
                                 float* ws, hipStream_t st);
hipError_t launch_state_scan(const PrefillPlan& p, const float* S, float* ws, hipStream_t st);
hipError_t launch_chunk_walk(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                             float* S, float* O, float* ws, hipStream_t st);

hipError_t launch_decode_step(lla_dtype dtype, const void* q, const void* k, const void* v,
                              int64_t BH, int dk, int dv, float* S, float* o, hipStream_t st);

// Gated (decayed) state, one gate per (b,h) and token (one query head per
// state): the prefill's segment pass, scan and walk (workspace: the segment
// states, then BH * n_seg floats of segment decays), and the decode step.
hipError_t launch_gated_prefill(const PrefillPlan& p, const void* Q, const void* K, const void* V,
                                const float* gate, float* S, float* O, float* ws, hipStream_t st);
hipError_t launch_decode_step_gated(lla_dtype dtype, const void* q, const void* k, const void* v,
                                    const float* gate, int64_t BH, int dk, int dv, float* S, float* o,
                                    hipStream_t st);

// Short prompts (T <= kDecodeTokensMax tokens, dk = dv in {64, 128}; with
// shared-state heads, T * group <= kDecodeTokensQueries) run as T fused decode
// steps with the state in registers; lla_prefill takes this route when
// decode_tokens_fit() holds.  One workgroup per key/value head.
constexpr int kDecodeTokensMax = 16;
constexpr int kDecodeTokensQueries = 64;
bool decode_tokens_fit(int64_t T, int dk, int dv, int64_t group);
hipError_t launch_decode_tokens(lla_dtype dtype, const void* q, const void* k, const void* v,
                                int64_t BHkv, int T, int group, int d, float* S, float* o,
                                bool zero_start, bool keep_state, hipStream_t st);
// Short continuations with shared-state heads on the matrix cores (bf16 or
// FP8 inputs, d in {64, 128}, T * group <= 64): one chunk of the walk per
// key/value head (k_tokens_grouped; k_tokens_grouped_pipe at d = 128).  Not
// the bits of T decode steps.  Used from kGroupedMatrixMinTokens tokens on:
// below that the fused decode steps
// are faster (their cost grows with T, this kernel's hardly does).
constexpr int kGroupedMatrixMinTokens = 8;
hipError_t launch_tokens_grouped(lla_dtype dtype, const void* q, const void* k, const void* v, int64_t BHkv,
                                 int T, int group, int d, float* S, float* o, bool zero_start, hipStream_t st);
// S += sum_{t < m} k_t v_t^T per key/value head (m = accepted[head / Hkv]
// clamped to [0, T], or T for a null accepted), with the decode step's
// per-element arithmetic; k, v: [BHkv][T][d].
hipError_t launch_state_commit(lla_dtype dtype, const void* k, const void* v, const int32_t* accepted,
                               int64_t BHkv, int Hkv, int T, int dk, int dv, float* S, hipStream_t st);
// The gated commit: S <- g_t S + k_t v_t^T for t < m (the gated decode
// step's arithmetic), gate: [BH][T]; H heads per sequence.
hipError_t launch_state_commit_gated(lla_dtype dtype, const void* k, const void* v, const float* gate,
                                     const int32_t* accepted, int64_t BH, int H, int T, int dk, int dv,
                                     float* S, hipStream_t st);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

// Shared-state heads: `group` query heads read each key/value state (any
// group >= 1, dk, dv <= 128).  q: [BHkv * group][dk], o: [BHkv * group][dv].
// The query rows are staged kDecodeGroupBatch at a time.
constexpr int kDecodeGroupMax = 16;  // largest group of the fused short continuations
constexpr int kDecodeGroupBatch = 16;
hipError_t launch_decode_group(lla_dtype dtype, const void* q, const void* k, const void* v,
                               int64_t BHkv, int group, int dk, int dv, float* S, float* o, hipStream_t st);
// The same with a decayed state: S = g S + k v^T, one gate per key/value head.
hipError_t launch_decode_group_gated(lla_dtype dtype, const void* q, const void* k, const void* v,
                                     const float* gate, int64_t BHkv, int group, int dk, int dv, float* S,
                                     float* o, hipStream_t st);

// lla_prefill_noalloc: the prefill workspace in a static device array of
// this many bytes per device (lla_noalloc.hip); *out = its address on the
// stream's device (the current device for the NULL stream), looked up on the
// first call per device.
constexpr size_t kNoAllocScratchBytes = LLA_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(hipStream_t stream, float** out);

}  // namespace lla
