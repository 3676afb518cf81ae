// lla_abi.cpp -- the C ABI of liblla: argument checking, planning and
// dispatch to the kernel launchers.  Every check runs on the host before any
// HIP call, so a rejected call touches no buffer and no device.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "lla.h"
#include "lla_internal.h"

namespace {

thread_local int g_last_device_error = 0;

constexpr int64_t kMaxHeadDim = 128;
constexpr int64_t kMaxChunkBf16 = 128;
constexpr int64_t kMaxChunkF32 = 64;
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

int64_t elem_size(lla_dtype dt) { return dt == LLA_FP8_E4M3 ? 1 : (dt == LLA_BF16 ? 2 : 4); }
bool known_dtype(int dt) { return dt == LLA_BF16 || dt == LLA_F32 || dt == LLA_FP8_E4M3; }

// Sizes shared by every call.  `C` < 0 means "no chunk size" (decode, init).
lla_status check_sizes(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C) {
    if (B < 1 || H < 1 || T < 0) return LLA_ERR_SHAPE;
    if (dk < 1 || dk > kMaxHeadDim || dv < 1 || dv > kMaxHeadDim) return LLA_ERR_SHAPE;
    if (B > kMaxStreams || H > kMaxStreams || B * H > kMaxStreams) return LLA_ERR_SHAPE;
    if (C >= 0 && (C < 1 || C > kMaxChunkBf16)) return LLA_ERR_SHAPE;
    // B*H*T*max(dk,dv)*4 bytes must be representable.
    const int64_t dmax = dk > dv ? dk : dv;
    if (T > 0 && B * H > (((int64_t)1 << 60) / T) / (dmax * 4)) return LLA_ERR_SHAPE;
    return LLA_OK;
}

lla_status check_dtype(int dt, int64_t C) {
    if (!known_dtype(dt)) return LLA_ERR_DTYPE;
    if (dt == LLA_F32 && C > kMaxChunkF32) return LLA_ERR_UNSUPPORTED;
    return LLA_OK;
}

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

size_t ws_bytes_for(const lla::PrefillPlan& p) {
    if (!p.use_ws) return 0;
    return (size_t)(p.BH * p.n_seg * (int64_t)p.dk * p.dv) * sizeof(float);
}

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
                         bool needs_o, bool needs_ws, lla_dtype dt, int64_t B, Heads h,
                         int64_t T, int64_t dk, int64_t dv, int64_t C, lla::PrefillPlan& plan) {
    lla_status st = check_heads(h);
    if (st != LLA_OK) return st;
    st = check_sizes(B, h.q, T, dk, dv, C);
    if (st != LLA_OK) return st;
    st = check_dtype((int)dt, C);
    if (st != LLA_OK) return st;
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
    const Span w = span((needs_ws && need_ws > 0) ? b.ws : nullptr, (int64_t)need_ws);
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
    switch (s) {
        case LLA_OK: return "ok";
        case LLA_ERR_NULL: return "a required pointer is NULL";
        case LLA_ERR_SHAPE: return "a size is out of range";
        case LLA_ERR_DTYPE: return "unknown dtype";
        case LLA_ERR_UNSUPPORTED: return "unsupported combination (fp32 inputs need C <= 64)";
        case LLA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case LLA_ERR_ALIAS: return "an output overlaps another buffer";
        case LLA_ERR_WORKSPACE: return "workspace missing or too small";
        case LLA_ERR_DEVICE: return "a HIP call failed";
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

size_t lla_prefill_workspace_size(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                  int64_t C) {
    return lla_prefill_gqa_workspace_size(B, H, H, T, dk, dv, C);
}

size_t lla_prefill_gqa_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk,
                                      int64_t dv, int64_t C) {
    if (check_heads(Heads{Hq, Hkv}) != LLA_OK || check_sizes(B, Hq, T, dk, dv, C) != LLA_OK) return 0;
    return ws_bytes_for(make_plan(LLA_BF16, B, Heads{Hq, Hkv}, T, dk, dv, C));
}

lla_status lla_prefill_segment_states(const void* K, const void* V, lla_dtype dtype, int64_t B,
                                      int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    lla::PrefillPlan p;
    PrefillBufs b{nullptr, K, V, nullptr, nullptr, nullptr, workspace, workspace_bytes};
    lla_status st = check_prefill(b, false, true, false, false, true, dtype, B, Heads{H, H}, T, dk, dv, C, p);
    if (st != LLA_OK || T == 0) return st;
    return device_status(lla::launch_segment_states(p, K, V, (float*)workspace, (hipStream_t)stream));
}

lla_status lla_prefill_state_scan(const float* S, int64_t B, int64_t H, int64_t T, int64_t dk,
                                  int64_t dv, int64_t C, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    lla::PrefillPlan p;
    PrefillBufs b{nullptr, nullptr, nullptr, S, nullptr, nullptr, workspace, workspace_bytes};
    lla_status st = check_prefill(b, false, false, true, false, true, LLA_BF16, B, Heads{H, H}, T, dk,
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
    lla_status st = check_prefill(b, true, true, true, true, true, dtype, B, Heads{H, H}, T, dk, dv, C, p);
    if (st != LLA_OK || T == 0) return st;
    return device_status(lla::launch_chunk_walk(p, Q, K, V, S, O, (float*)workspace, (hipStream_t)stream));
}

}  // extern "C"

namespace {

lla_status prefill_impl(const void* Q, const void* K, const void* V, lla_dtype dtype, int64_t B,
                        Heads h, int64_t T, int64_t dk, int64_t dv, int64_t C, unsigned flags,
                        float* S, float* O, void* workspace, size_t workspace_bytes, void* stream) {
    if (flags & ~(unsigned)LLA_PREFILL_ZERO_STATE) return LLA_ERR_UNSUPPORTED;
    const bool zero = (flags & LLA_PREFILL_ZERO_STATE) != 0;
    lla::PrefillPlan p;
    PrefillBufs b{Q, K, V, nullptr, S, O, workspace, workspace_bytes};
    lla_status st = check_prefill(b, true, true, true, true, true, dtype, B, h, T, dk, dv, C, p);
    if (st != LLA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (T == 0)  // S_T = S_0: untouched, or zero for a fresh prompt
        return zero ? device_status(lla::launch_fill_zero(S, p.BH * dk * dv, s)) : LLA_OK;
    p.zero_start = zero;
    if (lla::decode_tokens_fit(T, (int)dk, (int)dv, p.group))  // a short prompt: fused decode steps
        return device_status(lla::launch_decode_tokens(dtype, Q, K, V, p.BH, (int)T, p.group, (int)dk, S, O,
                                                       zero, s));
    float* ws = (float*)workspace;
    st = device_status(lla::launch_segment_states(p, K, V, ws, s));
    if (st != LLA_OK) return st;
    st = device_status(lla::launch_state_scan(p, S, ws, s));
    if (st != LLA_OK) return st;
    return device_status(lla::launch_chunk_walk(p, Q, K, V, S, O, ws, s));
}

lla_status decode_impl(const void* q, const void* k, const void* v, lla_dtype dtype, int64_t B,
                       Heads h, int64_t dk, int64_t dv, float* S, float* o, void* stream) {
    lla_status st = check_heads(h);
    if (st != LLA_OK) return st;
    st = check_sizes(B, h.q, 1, dk, dv, -1);
    if (st != LLA_OK) return st;
    if (!known_dtype(dtype)) return LLA_ERR_DTYPE;
    const int64_t group = h.q / h.kv;
    if (group > 1 && !lla::decode_group_fit(group, (int)dk, (int)dv)) return LLA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !S || !o) return LLA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S) || !aligned16(o))
        return LLA_ERR_ALIGN;
    const int64_t BHq = B * h.q, BHkv = B * h.kv, es = elem_size(dtype);
    const Span sq = span(q, BHq * dk * es), sk = span(k, BHkv * dk * es), sv = span(v, BHkv * dv * es);
    const Span ss = span(S, BHkv * dk * dv * 4), so = span(o, BHq * dv * 4);
    if (overlap(ss, sq) || overlap(ss, sk) || overlap(ss, sv) || overlap(ss, so) || overlap(so, sq) ||
        overlap(so, sk) || overlap(so, sv))
        return LLA_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (group > 1)
        return device_status(lla::launch_decode_group(dtype, q, k, v, BHkv, (int)group, (int)dk, S, o, s));
    return device_status(lla::launch_decode_step(dtype, q, k, v, BHkv, (int)dk, (int)dv, S, o, s));
}

}  // namespace

extern "C" {

lla_status lla_prefill(const void* Q, const void* K, const void* V, lla_dtype dtype, int64_t B,
                       int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C, float* S, float* O,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(Q, K, V, dtype, B, Heads{H, H}, T, dk, dv, C, 0u, S, O, workspace,
                        workspace_bytes, stream);
}

lla_status lla_prefill_gqa(const void* Q, const void* K, const void* V, lla_dtype dtype, int64_t B,
                           int64_t Hq, int64_t Hkv, int64_t T, int64_t dk, int64_t dv, int64_t C,
                           float* S, float* O, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(Q, K, V, dtype, B, Heads{Hq, Hkv}, T, dk, dv, C, 0u, S, O, workspace,
                        workspace_bytes, stream);
}

lla_status lla_prefill_ex(const void* Q, const void* K, const void* V, lla_dtype dtype, int64_t B,
                          int64_t Hq, int64_t Hkv, int64_t T, int64_t dk, int64_t dv, int64_t C,
                          unsigned flags, float* S, float* O, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return prefill_impl(Q, K, V, dtype, B, Heads{Hq, Hkv}, T, dk, dv, C, flags, S, O, workspace,
                        workspace_bytes, stream);
}

lla_status lla_decode_step(const void* q, const void* k, const void* v, lla_dtype dtype,
                           int64_t B, int64_t H, int64_t dk, int64_t dv, float* S, float* o,
                           void* stream) {
    return decode_impl(q, k, v, dtype, B, Heads{H, H}, dk, dv, S, o, stream);
}

lla_status lla_decode_step_gqa(const void* q, const void* k, const void* v, lla_dtype dtype,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t dk, int64_t dv, float* S,
                               float* o, void* stream) {
    return decode_impl(q, k, v, dtype, B, Heads{Hq, Hkv}, dk, dv, S, o, stream);
}

}  // extern "C"
