/*
 * lla.h -- causal linear attention, chunkwise-parallel prefill and decode step,
 * on AMD Instinct MI355X (gfx950).  C ABI of liblla.so.
 *
 * The method (slide deck "Chunking, causality, and parallel prefill"):
 *
 *   recurrence ("Naive recurrence"):      S_t = S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t
 *   chunk form ("Split into chunks", "Causal triangle",
 *               "Incoming and outgoing state"), chunk c of C tokens:
 *        O_c   = tril(Q_c K_c^T) V_c + Q_c S_c     (diagonal kept)
 *        S_c+1 = S_c + K_c^T V_c                   (the only serial hop)
 *   decode ("Mechanism map", decode line): one token, the triangle is 1x1;
 *        S <- S + k v^T  then  o = S^T q.
 *
 * No feature map, normaliser, 1/sqrt(d) scale or decay is applied: the deck's
 * trace uses raw q, k.  S is d_k x d_v with the key dimension as rows (the
 * deck's S_4 = K_1^T V_1 = [[3,4],[5,5]]).  The deck prints the inter-chunk
 * term as "K S_in"; its trace reads the state as q_t^T S_4 with q_t = k_t,
 * so the query is used: Q_c S_c.
 *
 * Conventions for every call
 * --------------------------
 * Layouts (dense, row-major, no strides):
 *   Q, K : [B][H][T][dk]      V : [B][H][T][dv]      (dtype: bf16, fp32 or FP8)
 *   O    : [B][H][T][dv]      fp32 output
 *   S    : [B][H][dk][dv]     fp32 recurrent state, row i = key dimension i
 *   decode: q, k : [B][H][dk]   v : [B][H][dv]   o : [B][H][dv] fp32
 * HIP graphs: the calls launch kernels only (no allocation, no memset node),
 * so they may be captured into a HIP graph on the capture stream; a replay
 * reuses the captured pointers, which must stay allocated.
 * Pointers are device pointers (HIP device memory of the current device),
 * 16-byte aligned.  The caller owns every buffer, including the workspace;
 * the library allocates nothing, holds no mutable global state and is safe
 * to call from several host threads on different streams.
 * `stream` is a hipStream_t (NULL = the default stream).  Every call only
 * enqueues work on that stream and returns without synchronising; results
 * are valid once the stream has been synchronised.
 * Limits: B, H >= 1; T >= 0 (T = 0 is a no-op that leaves S untouched);
 * 1 <= dk, dv <= 128; 1 <= C <= 128 for bf16 and FP8 inputs, 1 <= C <= 64 for
 * fp32 inputs; B*H <= 2^20 (H counts query heads in the grouped calls) and
 * B*H*T*max(dk,dv) <= 2^58, else LLA_ERR_SHAPE.  C need not divide T: the last
 * chunk of a sequence is shorter.
 * Errors: arguments are checked on the host before anything is enqueued; on
 * any error no buffer is touched and a status other than LLA_OK is returned.
 * LLA_ERR_DEVICE means the HIP launch itself failed (lla_last_device_error()
 * gives the hipError_t); faults inside a kernel surface at the caller's next
 * synchronisation.  The library never aborts, exits or prints.
 * Numerics: bf16 inputs are multiplied on bf16 matrix cores with fp32
 * accumulation; the fp32 state enters Q_c S_c as a sum of two bf16 parts
 * (high and low), and so do the masked scores entering P V for chunks of up
 * to 64 tokens (chunks of 128 round them to one bf16 value), so
 * integer-valued inputs whose partial sums stay below 2^16 in the state and
 * 2^24 elsewhere give exact results.  fp32 inputs use
 * fp32 matrix-core instructions throughout.  FP8 inputs (the 8-bit format
 * that the blog "A 128 000 tokens, l'attention avale 85 % du calcul" says the
 * attention measurements it reports use, for the arithmetic and the cache
 * alike) are the OCP E4M3 format: 1 sign, 4 exponent (bias 7) and 3
 * mantissa bits, subnormals, no infinities, NaN = S.1111.111 (torch's
 * float8_e4m3fn).  Every E4M3 value is exactly a bf16 value, so they are
 * decoded to bf16 on their way into LDS and take the bf16 path with the same
 * results as those values given in bf16.  No scale factor is applied: the
 * method is linear in each of q, k and v, so per-tensor scales s_q, s_k, s_v
 * fold into the outputs (O and the state's increment scale by s_q s_k s_v
 * and s_k s_v) and stay with the caller.  The state and O stay fp32.
 */
#ifndef LLA_H
#define LLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LLA_OK = 0,
    LLA_ERR_NULL = 1,        /* a required pointer is NULL */
    LLA_ERR_SHAPE = 2,       /* a size is out of range */
    LLA_ERR_DTYPE = 3,       /* unknown dtype */
    LLA_ERR_UNSUPPORTED = 4, /* valid request the library does not handle: fp32 with C > 64,
                                a grouped decode shape other than dk = dv in {64, 128} with
                                at most 16 query heads per group, unknown option bits */
    LLA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
    LLA_ERR_ALIAS = 6,       /* an output overlaps an input, another output or the workspace */
    LLA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than lla_prefill_workspace_size() */
    LLA_ERR_DEVICE = 8       /* a HIP call failed (see lla_last_device_error) */
} lla_status;

typedef enum {
    LLA_BF16 = 0,    /* bfloat16 Q/K/V (q/k/v) */
    LLA_F32 = 1,     /* float32 Q/K/V (q/k/v) */
    LLA_FP8_E4M3 = 2 /* OCP FP8 E4M3 Q/K/V (q/k/v), one byte per element */
} lla_dtype;

/* Short, static, human-readable name of a status code. */
const char *lla_status_string(lla_status s);

/* hipError_t of the last LLA_ERR_DEVICE on the calling host thread (0 if none). */
int lla_last_device_error(void);

/*
 * S = 0 for B*H states of dk x dv fp32: the fresh-prompt state S_0 = 0 of the
 * deck's worked trace.  Uses a fill kernel (no memset node), so it may be
 * captured into a HIP graph.
 */
lla_status lla_state_init(float *S, int64_t B, int64_t H, int64_t dk, int64_t dv,
                          void *stream);

/*
 * Number of consecutive chunks one workgroup walks in lla_prefill (a
 * "segment"); a sequence has ceil(ceil(T/C) / G) segments.  The choice
 * depends on the shape only (not on the device), so results are
 * reproducible across devices.  Returns 0 for invalid sizes.
 */
int64_t lla_prefill_segment_chunks(int64_t B, int64_t H, int64_t T, int64_t dk,
                                   int64_t dv, int64_t C);

/*
 * Bytes of device workspace lla_prefill needs for this shape: one fp32
 * dk x dv state per segment per (b, h) when a sequence has more than one
 * segment, else 0.  Returns 0 for invalid sizes as well.
 */
size_t lla_prefill_workspace_size(int64_t B, int64_t H, int64_t T, int64_t dk,
                                  int64_t dv, int64_t C);

/*
 * Chunkwise-parallel causal prefill (deck: "Split into chunks", "Causal
 * triangle", "Incoming and outgoing state", "Worked case - full trace").
 *
 * Q, K, V: inputs as above, `dtype` gives their element type.
 * S: in = S_0 (the incoming state, zero for a fresh prompt, or the state of a
 *    previous prefill/decode to continue a sequence); out = S_T.
 * O: out, o_t = S_t^T q_t for every token.
 * workspace: device buffer of at least lla_prefill_workspace_size() bytes
 *    (may be NULL when that size is 0).  Its content on return is the state
 *    at the start of every segment: state s of (b, h) -- [B][H][n_seg][dk][dv]
 *    fp32 -- holds S after s*G*C tokens (G = lla_prefill_segment_chunks).
 *
 * Enqueues up to three kernels on `stream`: per-segment K^T V, a scan over
 * segments, then the chunk walk (one workgroup per segment: per chunk the
 * masked score triangle, O_c, and the state hop).  Equivalent to calling
 * lla_prefill_segment_states, lla_prefill_state_scan and lla_prefill_chunks
 * in that order.
 *
 * Short prompts -- a few tokens continuing an existing state, where prefill
 * behaves like decode (deck: "Prefill and decode") -- take another route:
 * for 1 <= T <= 16 with dk = dv in {64, 128} (and, with shared-state heads,
 * T * G <= 64) the call runs T fused decode steps in one kernel (the state
 * read and written once, held in registers between the steps) with the
 * arithmetic of lla_decode_step (lla_decode_step_gqa), so its results equal T
 * successive decode-step calls bit for bit.  The workspace is not
 * touched on this route (it is still validated).
 */
lla_status lla_prefill(const void *Q, const void *K, const void *V, lla_dtype dtype,
                       int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t C,
                       float *S, float *O, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * Phase 1 of lla_prefill (deck: the outgoing state S_out = S_in + K_c^T V_c,
 * summed over a segment).  For every (b, h) and every segment s except the
 * last, writes K_s^T V_s (the segment's state increment) into workspace
 * slot s + 1.  No-op when a sequence has a single segment.
 */
lla_status lla_prefill_segment_states(const void *K, const void *V, lla_dtype dtype,
                                      int64_t B, int64_t H, int64_t T, int64_t dk,
                                      int64_t dv, int64_t C, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * Phase 2 of lla_prefill (deck: the serial chunk-to-chunk hop, "one hop
 * only").  Reads S_0 from S and the increments of phase 1; writes slot 0 =
 * S_0 and slot s = S_0 + sum of the increments of segments < s.  S is only
 * read.  No-op when a sequence has a single segment.
 */
lla_status lla_prefill_state_scan(const float *S, int64_t B, int64_t H, int64_t T,
                                  int64_t dk, int64_t dv, int64_t C, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Phase 3 of lla_prefill: every segment walks its chunks from its starting
 * state (slot s of the workspace, or S itself when there is one segment),
 * writing O_c = tril(Q_c K_c^T) V_c + Q_c S_c and advancing the state by
 * K_c^T V_c; the last segment writes S_T into S.
 */
lla_status lla_prefill_chunks(const void *Q, const void *K, const void *V, lla_dtype dtype,
                              int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                              int64_t C, float *S, float *O, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * One decode step for B*H sequences (deck: decode is the 1x1-triangle case;
 * what remains is the state read after the rank-1 update).
 * q, k: [B][H][dk]; v: [B][H][dv] (dtype); S: [B][H][dk][dv] fp32, updated in
 * place to S + k v^T; o: [B][H][dv] fp32 = (S + k v^T)^T q.
 */
lla_status lla_decode_step(const void *q, const void *k, const void *v, lla_dtype dtype,
                           int64_t B, int64_t H, int64_t dk, int64_t dv, float *S, float *o,
                           void *stream);

/*
 * Shared-state heads.  Hq query heads are grouped on Hkv key/value heads
 * (group size G = Hq / Hkv; query head h reads key/value head h / G), as in
 * grouped-query attention (blog "A 128 000 tokens, l'attention avale 85 % du
 * calcul", section on sharing heads to lighten memory).  Every key/value head
 * carries one state, updated once per token; each query head of its group
 * reads it:  S_t = S_{t-1} + k_t v_t^T,  o_t^(h) = S_t^T q_t^(h).
 *
 * Layouts: Q, O as lla_prefill with Hq heads; K, V and S as lla_prefill with
 * Hkv heads.  Conditions: 1 <= Hkv <= Hq, Hq a multiple of Hkv (else
 * LLA_ERR_SHAPE); the rest as lla_prefill.  With Hq = Hkv these are
 * lla_prefill and lla_prefill_workspace_size.  The per-segment K^T V and the
 * segment scan run once per key/value head; each query head's walk reads
 * them.  When G > 1 the walks always start from the workspace (which then
 * holds at least one state per key/value head).  Short prompts with
 * T * G <= 64 take the fused decode-step route described at lla_prefill.
 */
size_t lla_prefill_gqa_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                                      int64_t dk, int64_t dv, int64_t C);

lla_status lla_prefill_gqa(const void *Q, const void *K, const void *V, lla_dtype dtype,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk,
                           int64_t dv, int64_t C, float *S, float *O, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Options of lla_prefill_ex.
 *   LLA_PREFILL_ZERO_STATE: a fresh prompt.  The prefill starts from S_0 = 0
 *     (the deck's worked trace starts from zero) without reading S, which is
 *     output only and receives S_T; for T = 0, S is set to zero.  Saves the
 *     lla_state_init call and the read of S_0.
 */
#define LLA_PREFILL_ZERO_STATE 1u

/*
 * lla_prefill_gqa with options (a bitwise OR of LLA_PREFILL_* values, 0 for
 * none); unknown bits give LLA_ERR_UNSUPPORTED.  With flags = 0 and Hq = Hkv
 * this is lla_prefill; the workspace is that of lla_prefill_gqa_workspace_size.
 * Results with LLA_PREFILL_ZERO_STATE equal those of lla_state_init followed
 * by the call without it, bit for bit.
 */
lla_status lla_prefill_ex(const void *Q, const void *K, const void *V, lla_dtype dtype,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk,
                          int64_t dv, int64_t C, unsigned flags, float *S, float *O,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step with shared-state heads: q: [B][Hq][dk], k: [B][Hkv][dk],
 * v: [B][Hkv][dv] (dtype); S: [B][Hkv][dk][dv] fp32 updated once in place;
 * o: [B][Hq][dv] fp32.  Each state is read from memory once for the G query
 * heads of its group.  For G > 1 the library needs dk = dv in {64, 128} and
 * G <= 16 (else LLA_ERR_UNSUPPORTED); G = 1 is lla_decode_step.  Per query
 * head the arithmetic is that of lla_decode_step (identical bits).
 */
lla_status lla_decode_step_gqa(const void *q, const void *k, const void *v, lla_dtype dtype,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t dk, int64_t dv,
                               float *S, float *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H */
