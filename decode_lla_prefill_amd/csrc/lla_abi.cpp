// lla_abi.cpp -- the C ABI of liblla: argument checking, planning and
// dispatch to the kernel launchers.  Every check runs on the host before any
// HIP call, so a rejected call touches no buffer and no device.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <random>

#include "lla.h"
#include "lla_internal.h"

namespace {

thread_local int g_last_device_error = 0;

constexpr int64_t kMaxHeadDim = 128;
constexpr int64_t kMaxChunk = 128;
// B*H bound: every launch grid stays far below 2^32 work-items.
constexpr int64_t kMaxStreams = (int64_t)1 << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Span{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
bool overlap(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

// The int a caller passed for an enum parameter.  C lets any int through an
// enum; C++ may assume an enum object holds only values in its enumerators'
// range, so such a parameter is read as raw bytes and checked before it is
// used as the enum.
template <typename E>
int raw_enum(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "the C enums are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

int64_t elem_size(lla_dtype dt) { return dt == LLA_FP8_E4M3 ? 1 : (dt == LLA_BF16 ? 2 : 4); }
bool known_dtype(int dt) { return dt == LLA_BF16 || dt == LLA_F32 || dt == LLA_FP8_E4M3; }
constexpr unsigned kKnownFlags = LLA_PREFILL_ZERO_STATE | LLA_PREFILL_KEEP_STATE;

// Sizes shared by every call.  `C` < 0 means "no chunk size" (decode, init).
lla_status check_sizes(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C) {
    if (B < 1 || H < 1 || T < 0) return LLA_ERR_SHAPE;
    if (dk < 1 || dk > kMaxHeadDim || dv < 1 || dv > kMaxHeadDim) return LLA_ERR_SHAPE;
    if (B > kMaxStreams || H > kMaxStreams || B * H > kMaxStreams) return LLA_ERR_SHAPE;
    if (C >= 0 && (C < 1 || C > kMaxChunk)) return LLA_ERR_SHAPE;
    // B*H*T*max(dk,dv)*4 bytes must be representable.
    const int64_t dmax = dk > dv ? dk : dv;
    if (T > 0 && B * H > (((int64_t)1 << 60) / T) / (dmax * 4)) return LLA_ERR_SHAPE;
    return LLA_OK;
}

lla_status check_dtype(int dt) { return known_dtype(dt) ? LLA_OK : LLA_ERR_DTYPE; }

lla_status device_status(hipError_t e) {
    if (e == hipSuccess) return LLA_OK;
    g_last_device_error = (int)e;
    return LLA_ERR_DEVICE;
}

// Query heads Hq and key/value heads Hkv (Hq = Hkv without grouping).
struct Heads {
    int64_t q, kv;
};

// Head counts: 1 <= Hkv <= Hq, Hq a multiple of Hkv.
lla_status check_heads(Heads h) {
    if (h.q < 1 || h.kv < 1 || h.kv > h.q || h.q % h.kv != 0) return LLA_ERR_SHAPE;
    return LLA_OK;
}

lla::PrefillPlan make_plan(lla_dtype dt, int64_t B, Heads h, int64_t T, int64_t dk, int64_t dv,
                           int64_t C) {
    lla::PrefillPlan p{};
    p.B = B;
    p.H = h.q;
    p.Hkv = h.kv;
    p.T = T;
    p.dk = (int)dk;
    p.dv = (int)dv;
    p.C = (int)C;
    p.dtype = dt;
    lla::plan_prefill(p);
    return p;
}

// The workspace a prefill requires (what the arguments are checked against).
size_t ws_bytes_for(const lla::PrefillPlan& p) {
    if (!p.use_ws) return 0;
    return (size_t)(p.BH * p.n_seg * (int64_t)p.dk * p.dv) * sizeof(float);
}

// The workspace size the library reports: the required one, and for shapes
// that can run as one launch also room for its published segment sums (with
// less, that route sums every earlier segment itself).
size_t ws_bytes_reported(const lla::PrefillPlan& p) {
    const size_t need = ws_bytes_for(p);
    if (need == 0 || !lla::prefix_capable(p)) return need;
    const size_t pub = lla::prefix_publish_bytes(p);
    return need > pub ? need : pub;
}

// A flag value for one call's published segment sums: a Weyl sequence (odd
// step, so 2^64 calls before a repeat) from a seed drawn once per process,
// never 0.  A flag left in the workspace by an earlier call never equals a
// later call's token, so no clearing is needed between calls.
unsigned long long next_token() {
    static std::atomic<unsigned long long> state{[] {
        std::random_device rd;
        return ((unsigned long long)rd() << 32) ^ (unsigned long long)rd() ^
               (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    }()};
    unsigned long long t;
    do {
        t = state.fetch_add(0x9E3779B97F4A7C15ull, std::memory_order_relaxed) + 0x9E3779B97F4A7C15ull;
    } while (t == 0);
    return t;
}

std::atomic<uint64_t> g_publish_wait{lla::kPublishWaitTicks};

// Published sums need a fresh token per execution, which a captured launch
// (replayed with the arguments of its capture) does not get: on a stream
// that is capturing, the one-launch walk sums every earlier segment itself.
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

// The gated prefill's workspace: the segment states, then one decay (float)
// per (b,h) and segment; none with a single segment.
size_t gated_ws_bytes_for(const lla::PrefillPlan& p) {
    // grouped heads stage their start states even for a single segment
    if (p.n_seg <= 1 && p.group <= 1) return 0;
    return (size_t)(p.BH * p.n_seg * ((int64_t)p.dk * p.dv + 1)) * sizeof(float);
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Which buffers a prefill phase touches; null entries are not used.
struct PrefillBufs {
    const void *Q, *K, *V;
    const float* S_in;  // read only
    float* S_out;       // written
    float* O;
    void* ws;
    size_t ws_bytes;
};

lla_status check_prefill(const PrefillBufs& b, bool needs_q, bool needs_kv, bool needs_s,
                         bool needs_o, bool needs_ws, int dt_raw, int64_t B, Heads h,
                         int64_t T, int64_t dk, int64_t dv, int64_t C, lla::PrefillPlan& plan) {
    lla_status st = check_heads(h);
    if (st != LLA_OK) return st;
    st = check_sizes(B, h.q, T, dk, dv, C);
    if (st != LLA_OK) return st;
    st = check_dtype(dt_raw);
    if (st != LLA_OK) return st;
    const lla_dtype dt = (lla_dtype)dt_raw;
    plan = make_plan(dt, B, h, T, dk, dv, C);
    const bool empty = T == 0;
    // Pointers: Q/K/V/O may be NULL only for an empty prompt; S never.
    if (needs_q && !empty && !b.Q) return LLA_ERR_NULL;
    if (needs_kv && !empty && (!b.K || !b.V)) return LLA_ERR_NULL;
    if (needs_o && !empty && !b.O) return LLA_ERR_NULL;
    if (needs_s && !(b.S_in || b.S_out)) return LLA_ERR_NULL;
    const size_t need_ws = ws_bytes_for(plan);
    if (needs_ws && need_ws > 0 && (!b.ws || b.ws_bytes < need_ws)) return LLA_ERR_WORKSPACE;
    const void* ptrs[] = {needs_q ? b.Q : nullptr, needs_kv ? b.K : nullptr,
                          needs_kv ? b.V : nullptr, needs_s ? (const void*)b.S_in : nullptr,
                          needs_s ? (const void*)b.S_out : nullptr, needs_o ? (const void*)b.O : nullptr,
                          (needs_ws && need_ws > 0) ? b.ws : nullptr};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return LLA_ERR_ALIGN;
    if (empty) return LLA_OK;
    const int64_t es = elem_size(dt);
    const int64_t BHq = B * h.q, BHkv = B * h.kv;
    const Span q = span(needs_q ? b.Q : nullptr, needs_q ? BHq * T * dk * es : 0);
    const Span k = span(needs_kv ? b.K : nullptr, needs_kv ? BHkv * T * dk * es : 0);
    const Span v = span(needs_kv ? b.V : nullptr, needs_kv ? BHkv * T * dv * es : 0);
    const Span o = span(needs_o ? b.O : nullptr, needs_o ? BHq * T * dv * 4 : 0);
    const void* s_ptr = b.S_out ? (const void*)b.S_out : (const void*)b.S_in;
    const Span s = span(needs_s ? s_ptr : nullptr, needs_s ? BHkv * dk * dv * 4 : 0);
    // (a one-launch walk given room for its published sums writes them too)
    size_t used_ws = need_ws;
    if (need_ws > 0 && lla::prefix_capable(plan) && b.ws_bytes >= lla::prefix_publish_bytes(plan))
        used_ws = std::max(used_ws, lla::prefix_publish_bytes(plan));
    const Span w = span((needs_ws && need_ws > 0) ? b.ws : nullptr, (int64_t)used_ws);
    // Outputs (O, S when written, the workspace) must not overlap anything else.
    const Span all[] = {q, k, v, o, s, w};
    const int outs[] = {3, b.S_out ? 4 : -1, 5};
    for (int oi : outs) {
        if (oi < 0) continue;
        for (int c = 0; c < 6; ++c)
            if (c != oi && overlap(all[oi], all[c])) return LLA_ERR_ALIAS;
    }
    return LLA_OK;
}

}  // namespace

extern "C" {

const char* lla_status_string(lla_status s) {
    switch (raw_enum(s)) {
        case LLA_OK: return "ok";
        case LLA_ERR_NULL: return "a required pointer is NULL";
        case LLA_ERR_SHAPE: return "a size is out of range";
        case LLA_ERR_DTYPE: return "unknown dtype";
        case LLA_ERR_UNSUPPORTED:
            return "unsupported request (unknown option bits)";
        case LLA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case LLA_ERR_ALIAS: return "an output overlaps another buffer";
        case LLA_ERR_WORKSPACE: return "workspace missing or too small";
        case LLA_ERR_DEVICE: return "a HIP call failed";
        case LLA_ERR_SCRATCH: return "the shape needs more workspace than the static scratch array holds";
    }
    return "unknown status";
}

int lla_last_device_error(void) { return g_last_device_error; }

lla_status lla_state_init(float* S, int64_t B, int64_t H, int64_t dk, int64_t dv, void* stream) {
    lla_status st = check_sizes(B, H, 0, dk, dv, -1);
    if (st != LLA_OK) return st;
    if (!S) return LLA_ERR_NULL;
    if (!aligned16(S)) return LLA_ERR_ALIGN;
    return device_status(lla::launch_fill_zero(S, B * H * dk * dv, (hipStream_t)stream));
}

int64_t lla_prefill_segment_chunks(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                   int64_t C) {
    if (check_sizes(B, H, T, dk, dv, C) != LLA_OK) return 0;
    return make_plan(LLA_BF16, B, Heads{H, H}, T, dk, dv, C).G;
}

lla_status lla_set_publish_wait_ticks(int64_t ticks) {
    if (ticks < 0) return LLA_ERR_SHAPE;
    g_publish_wait.store((uint64_t)ticks, std::memory_order_relaxed);
    return LLA_OK;
}

size_t lla_prefill_workspace_size(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                  int64_t C) {
    return lla_prefill_gqa_workspace_size(B, H, H, T, dk, dv, C);
}

size_t lla_prefill_gqa_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk,
                                      int64_t dv, int64_t C) {
    if (check_heads(Heads{Hq, Hkv}) != LLA_OK || check_sizes(B, Hq, T, dk, dv, C) != LLA_OK) return 0;
    return ws_bytes_reported(make_plan(LLA_BF16, B, Heads{Hq, Hkv}, T, dk, dv, C));
}

lla_status lla_prefill_segment_states(const void* K, const void* V, lla_dtype dtype, int64_t B,
                                      int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    lla::PrefillPlan p;
    PrefillBufs b{nullptr, K, V, nullptr, nullptr, nullptr, workspace, workspace_bytes};
    lla_status st = check_prefill(b, false, true, false, false, true, raw_enum(dtype), B, Heads{H, H}, T, dk,
                                  dv, C, p);
    if (st != LLA_OK || T == 0) return st;
    return device_status(lla::launch_segment_states(p, K, V, (float*)workspace, (hipStream_t)stream));
}

lla_status lla_prefill_state_scan(const float* S, int64_t B, int64_t H, int64_t T, int64_t dk,
                                  int64_t dv, int64_t C, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    lla::PrefillPlan p;
    PrefillBufs b{nullptr, nullptr, nullptr, S, nullptr, nullptr, workspace, workspace_bytes};
    lla_status st = check_prefill(b, false, false, true, false, true, (int)LLA_BF16, B, Heads{H, H}, T, dk,
                                  dv, C, p);
    if (st != LLA_OK || T == 0) return st;
    return device_status(lla::launch_state_scan(p, S, (float*)workspace, (hipStream_t)stream));
}

lla_status lla_prefill_chunks(const void* Q, const void* K, const void* V, lla_dtype dtype,
                              int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C,
                              float* S, float* O, void* workspace, size_t workspace_bytes,
                              void* stream) {
    lla::PrefillPlan p;
    PrefillBufs b{Q, K, V, nullptr, S, O, workspace, workspace_bytes};
    lla_status st = check_prefill(b, true, true, true, true, true, raw_enum(dtype), B, Heads{H, H}, T, dk,
                                  dv, C, p);
    if (st != LLA_OK || T == 0) return st;
    return device_status(lla::launch_chunk_walk(p, Q, K, V, S, O, (float*)workspace, (hipStream_t)stream));
}

}  // extern "C"

namespace {

lla_status prefill_impl(const void* Q, const void* K, const void* V, int dt_raw, int64_t B,
                        Heads h, int64_t T, int64_t dk, int64_t dv, int64_t C, unsigned flags,
                        float* S, float* O, void* workspace, size_t workspace_bytes, void* stream) {
    if (flags & ~kKnownFlags) return LLA_ERR_UNSUPPORTED;
    const bool zero = (flags & LLA_PREFILL_ZERO_STATE) != 0;
    const bool keep = (flags & LLA_PREFILL_KEEP_STATE) != 0;
    lla::PrefillPlan p;
    PrefillBufs b{Q, K, V, nullptr, S, O, workspace, workspace_bytes};
    lla_status st = check_prefill(b, true, true, true, true, true, dt_raw, B, h, T, dk, dv, C, p);
    if (st != LLA_OK) return st;
    const lla_dtype dtype = (lla_dtype)dt_raw;  // checked
    hipStream_t s = (hipStream_t)stream;
    const bool fused = lla::decode_tokens_fit(T, (int)dk, (int)dv, p.group);
    if (T == 0)  // S_T = S_0: untouched, or zero for a fresh prompt (never written with KEEP_STATE)
        return zero && !keep ? device_status(lla::launch_fill_zero(S, p.BH * dk * dv, s)) : LLA_OK;
    p.zero_start = zero;
    p.keep = keep;
    if (fused) {  // a short prompt
        // Several query heads per state (bf16 or FP8) and at least 8 tokens:
        // one chunk on the matrix cores; otherwise, and for a verify pass,
        // fused decode steps (the bits of T decode steps).
        if (p.group > 1 && T >= lla::kGroupedMatrixMinTokens && !keep && dtype != LLA_F32)
            return device_status(lla::launch_tokens_grouped(dtype, Q, K, V, p.BH, (int)T, p.group, (int)dk, S,
                                                            O, zero, s));
        return device_status(lla::launch_decode_tokens(dtype, Q, K, V, p.BH, (int)T, p.group, (int)dk, S, O,
                                                       zero, keep, s));
    }
    float* ws = (float*)workspace;
    const bool can_publish = ws && workspace_bytes >= lla::prefix_publish_bytes(p) && !capturing(s);
    p.prefix = lla::prefix_walk_fits(p, can_publish);
    if (p.prefix && can_publish) {
        p.publish = true;
        p.token = next_token();
        p.wait_ticks = g_publish_wait.load(std::memory_order_relaxed);
    }
    if (!p.prefix) {
        st = device_status(lla::launch_segment_states(p, K, V, ws, s));
        if (st != LLA_OK) return st;
        st = device_status(lla::launch_state_scan(p, S, ws, s));
        if (st != LLA_OK) return st;
    }
    return device_status(lla::launch_chunk_walk(p, Q, K, V, S, O, ws, s));
}

// gate: null, or one gate per state (the gated step), [B][Hkv].
lla_status decode_impl(const void* q, const void* k, const void* v, int dt_raw, int64_t B,
                       Heads h, int64_t dk, int64_t dv, float* S, float* o, void* stream,
                       const float* gate = nullptr, bool gated = false) {
    lla_status st = check_heads(h);
    if (st != LLA_OK) return st;
    st = check_sizes(B, h.q, 1, dk, dv, -1);
    if (st != LLA_OK) return st;
    if (!known_dtype(dt_raw)) return LLA_ERR_DTYPE;
    const lla_dtype dtype = (lla_dtype)dt_raw;
    const int64_t group = h.q / h.kv;
    if (!q || !k || !v || !S || !o || (gated && !gate)) return LLA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S) || !aligned16(o) ||
        (gated && !aligned4(gate)))
        return LLA_ERR_ALIGN;
    const int64_t BHq = B * h.q, BHkv = B * h.kv, es = elem_size(dtype);
    const Span sq = span(q, BHq * dk * es), sk = span(k, BHkv * dk * es), sv = span(v, BHkv * dv * es);
    const Span ss = span(S, BHkv * dk * dv * 4), so = span(o, BHq * dv * 4);
    if (overlap(ss, sq) || overlap(ss, sk) || overlap(ss, sv) || overlap(ss, so) || overlap(so, sq) ||
        overlap(so, sk) || overlap(so, sv))
        return LLA_ERR_ALIAS;
    if (gated) {  // one gate per state
        const Span sg = span(gate, BHkv * 4);
        if (overlap(ss, sg) || overlap(so, sg)) return LLA_ERR_ALIAS;
    }
    hipStream_t s = (hipStream_t)stream;
    if (gated && group > 1)
        return device_status(lla::launch_decode_group_gated(dtype, q, k, v, gate, BHkv, (int)group, (int)dk,
                                                            (int)dv, S, o, s));
    if (gated)
        return device_status(lla::launch_decode_step_gated(dtype, q, k, v, gate, BHkv, (int)dk, (int)dv, S, o, s));
    if (group > 1)
        return device_status(lla::launch_decode_group(dtype, q, k, v, BHkv, (int)group, (int)dk, (int)dv, S, o,
                                                                s));
    return device_status(lla::launch_decode_step(dtype, q, k, v, BHkv, (int)dk, (int)dv, S, o, s));
}

// lla_state_commit and lla_state_commit_gated (gate non-null only for the latter).
lla_status commit_impl(const void* K, const void* V, const float* gate, bool gated, int dt_raw, int64_t B,
                       int64_t H, int64_t T, int64_t dk, int64_t dv, const int32_t* accepted, float* S,
                       void* stream) {
    lla_status st = check_sizes(B, H, T, dk, dv, -1);
    if (st != LLA_OK) return st;
    if (!known_dtype(dt_raw)) return LLA_ERR_DTYPE;
    if (!S || (T > 0 && (!K || !V || (gated && !gate)))) return LLA_ERR_NULL;
    if (!aligned16(S) || (T > 0 && (!aligned16(K) || !aligned16(V))) || (accepted && !aligned16(accepted)) ||
        (gated && T > 0 && !aligned4(gate)))
        return LLA_ERR_ALIGN;
    if (T == 0) return LLA_OK;
    const int64_t es = elem_size((lla_dtype)dt_raw);
    const Span ss = span(S, B * H * dk * dv * 4), sk = span(K, B * H * T * dk * es),
               sv = span(V, B * H * T * dv * es), sa = span(accepted, accepted ? B * 4 : 0),
               sg = span(gated ? gate : nullptr, gated ? B * H * T * 4 : 0);
    if (overlap(ss, sk) || overlap(ss, sv) || overlap(ss, sa) || overlap(ss, sg)) return LLA_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (gated)
        return device_status(lla::launch_state_commit_gated((lla_dtype)dt_raw, K, V, gate, accepted, B * H, (int)H,
                                                            (int)T, (int)dk, (int)dv, S, s));
    return device_status(lla::launch_state_commit((lla_dtype)dt_raw, K, V, accepted, B * H, (int)H, (int)T,
                                                  (int)dk, (int)dv, S, s));
}

// lla_prefill_gated(_gqa); the dtype as its raw integer (a C caller may pass
// any int, which the C++ enum need not hold).
lla_status gated_prefill_impl(const void* Q, const void* K, const void* V, const float* gate, int dt_raw,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk, int64_t dv, int64_t C,
                              unsigned flags, float* S, float* O, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (flags & ~kKnownFlags) return LLA_ERR_UNSUPPORTED;
    const bool zero = (flags & LLA_PREFILL_ZERO_STATE) != 0;
    const bool keep = (flags & LLA_PREFILL_KEEP_STATE) != 0;
    lla::PrefillPlan p;
    PrefillBufs b{Q, K, V, nullptr, S, O, nullptr, 0};
    lla_status st = check_prefill(b, true, true, true, true, false, dt_raw, B, Heads{Hq, Hkv}, T, dk, dv,
                                  C, p);
    if (st != LLA_OK) return st;
    const size_t need = gated_ws_bytes_for(p);
    if (T > 0 && !gate) return LLA_ERR_NULL;
    if (need > 0 && (!workspace || workspace_bytes < need)) return LLA_ERR_WORKSPACE;
    if ((T > 0 && !aligned4(gate)) || (need > 0 && !aligned16(workspace))) return LLA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (T == 0) return zero && !keep ? device_status(lla::launch_fill_zero(S, B * Hkv * dk * dv, s)) : LLA_OK;
    // The gate is read only; the workspace is written: neither may overlap an
    // output, and the workspace nothing at all.
    const int64_t BHq = B * Hq, BHkv = B * Hkv, es = elem_size((lla_dtype)dt_raw);
    const Span sq = span(Q, BHq * T * dk * es), sk = span(K, BHkv * T * dk * es), sv = span(V, BHkv * T * dv * es);
    const Span so = span(O, BHq * T * dv * 4), ss = span(S, BHkv * dk * dv * 4), sg = span(gate, BHkv * T * 4);
    const Span sw = span(need > 0 ? workspace : nullptr, (int64_t)need);
    if (overlap(so, sg) || overlap(ss, sg)) return LLA_ERR_ALIAS;
    for (Span x : {sq, sk, sv, so, ss, sg})
        if (overlap(sw, x)) return LLA_ERR_ALIAS;
    p.zero_start = zero;
    p.keep = keep;
    p.use_ws = need > 0;
    return device_status(lla::launch_gated_prefill(p, Q, K, V, gate, S, O, (float*)workspace, s));
}


}  // namespace

extern "C" {

lla_status lla_prefill(const void* Q, const void* K, const void* V, lla_dtype dtype, int64_t B,
                       int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C, float* S, float* O,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(Q, K, V, raw_enum(dtype), B, Heads{H, H}, T, dk, dv, C, 0u, S, O, workspace,
                        workspace_bytes, stream);
}

lla_status lla_prefill_gqa(const void* Q, const void* K, const void* V, lla_dtype dtype, int64_t B,
                           int64_t Hq, int64_t Hkv, int64_t T, int64_t dk, int64_t dv, int64_t C,
                           float* S, float* O, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(Q, K, V, raw_enum(dtype), B, Heads{Hq, Hkv}, T, dk, dv, C, 0u, S, O, workspace,
                        workspace_bytes, stream);
}

lla_status lla_prefill_ex(const void* Q, const void* K, const void* V, lla_dtype dtype, int64_t B,
                          int64_t Hq, int64_t Hkv, int64_t T, int64_t dk, int64_t dv, int64_t C,
                          unsigned flags, float* S, float* O, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return prefill_impl(Q, K, V, raw_enum(dtype), B, Heads{Hq, Hkv}, T, dk, dv, C, flags, S, O, workspace,
                        workspace_bytes, stream);
}

lla_status lla_prefill_noalloc(const void* Q, const void* K, const void* V, lla_dtype dtype, int64_t B,
                               int64_t Hq, int64_t Hkv, int64_t T, int64_t dk, int64_t dv, int64_t C,
                               unsigned flags, float* S, float* O, void* stream) {
    // Everything but the workspace is checked first (no HIP call), then the
    // workspace the plan needs against the static array's size.
    if (flags & ~kKnownFlags) return LLA_ERR_UNSUPPORTED;
    lla::PrefillPlan p;
    PrefillBufs b{Q, K, V, nullptr, S, O, nullptr, 0};
    lla_status st = check_prefill(b, true, true, true, true, false, raw_enum(dtype), B, Heads{Hq, Hkv}, T, dk,
                                  dv, C, p);
    if (st != LLA_OK) return st;
    const size_t need = ws_bytes_for(p);
    if (need > lla::kNoAllocScratchBytes) return LLA_ERR_SCRATCH;
    float* ws = nullptr;
    if (T > 0 && need > 0) {
        st = device_status(lla::noalloc_scratch((hipStream_t)stream, &ws));
        if (st != LLA_OK) return st;
    }
    return prefill_impl(Q, K, V, raw_enum(dtype), B, Heads{Hq, Hkv}, T, dk, dv, C, flags, S, O, ws,
                        ws ? lla::kNoAllocScratchBytes : 0, stream);
}

lla_status lla_state_commit(const void* K, const void* V, lla_dtype dtype, int64_t B, int64_t H,
                            int64_t T, int64_t dk, int64_t dv, const int32_t* accepted, float* S,
                            void* stream) {
    return commit_impl(K, V, nullptr, false, raw_enum(dtype), B, H, T, dk, dv, accepted, S, stream);
}

lla_status lla_state_commit_gated(const void* K, const void* V, const float* gate, lla_dtype dtype, int64_t B,
                                  int64_t H, int64_t T, int64_t dk, int64_t dv, const int32_t* accepted,
                                  float* S, void* stream) {
    return commit_impl(K, V, gate, true, raw_enum(dtype), B, H, T, dk, dv, accepted, S, stream);
}

lla_status lla_decode_step(const void* q, const void* k, const void* v, lla_dtype dtype,
                           int64_t B, int64_t H, int64_t dk, int64_t dv, float* S, float* o,
                           void* stream) {
    return decode_impl(q, k, v, raw_enum(dtype), B, Heads{H, H}, dk, dv, S, o, stream);
}

lla_status lla_decode_step_gqa(const void* q, const void* k, const void* v, lla_dtype dtype,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t dk, int64_t dv, float* S,
                               float* o, void* stream) {
    return decode_impl(q, k, v, raw_enum(dtype), B, Heads{Hq, Hkv}, dk, dv, S, o, stream);
}

size_t lla_prefill_gated_workspace_size(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C) {
    return lla_prefill_gated_gqa_workspace_size(B, H, H, T, dk, dv, C);
}

size_t lla_prefill_gated_gqa_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk, int64_t dv,
                                            int64_t C) {
    if (check_heads(Heads{Hq, Hkv}) != LLA_OK || check_sizes(B, Hq, T, dk, dv, C) != LLA_OK) return 0;
    return gated_ws_bytes_for(make_plan(LLA_BF16, B, Heads{Hq, Hkv}, T, dk, dv, C));
}

lla_status lla_prefill_gated(const void* Q, const void* K, const void* V, const float* gate, lla_dtype dtype,
                             int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C, unsigned flags,
                             float* S, float* O, void* workspace, size_t workspace_bytes, void* stream) {
    return gated_prefill_impl(Q, K, V, gate, raw_enum(dtype), B, H, H, T, dk, dv, C, flags, S, O, workspace,
                              workspace_bytes, stream);
}

lla_status lla_prefill_gated_gqa(const void* Q, const void* K, const void* V, const float* gate, lla_dtype dtype,
                                 int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk, int64_t dv, int64_t C,
                                 unsigned flags, float* S, float* O, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return gated_prefill_impl(Q, K, V, gate, raw_enum(dtype), B, Hq, Hkv, T, dk, dv, C, flags, S, O, workspace,
                              workspace_bytes, stream);
}

lla_status lla_decode_step_gated(const void* q, const void* k, const void* v, const float* gate,
                                 lla_dtype dtype, int64_t B, int64_t H, int64_t dk, int64_t dv, float* S,
                                 float* o, void* stream) {
    return decode_impl(q, k, v, raw_enum(dtype), B, Heads{H, H}, dk, dv, S, o, stream, gate, true);
}

lla_status lla_decode_step_gated_gqa(const void* q, const void* k, const void* v, const float* gate,
                                     lla_dtype dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t dk, int64_t dv,
                                     float* S, float* o, void* stream) {
    return decode_impl(q, k, v, raw_enum(dtype), B, Heads{Hq, Hkv}, dk, dv, S, o, stream, gate, true);
}

}  // extern "C"
