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
 * 1 <= dk, dv <= 128; 1 <= C <= 128; B*H <= 2^20 (H counts query heads in the grouped calls) and
 * B*H*T*max(dk,dv) <= 2^58, else LLA_ERR_SHAPE.  C need not divide T: the last
 * chunk of a sequence is shorter.  The library runs chunks of C > 64 tokens as
 * two chunks of c = ceil(C/2) tokens each (c = C for C <= 64): the chunk form
 * gives the same result for any chunk size, up to rounding.
 * Errors: arguments are checked on the host before anything is enqueued; on
 * any error no buffer is touched and a status other than LLA_OK is returned.
 * LLA_ERR_DEVICE means the HIP launch itself failed (lla_last_device_error()
 * gives the hipError_t); faults inside a kernel surface at the caller's next
 * synchronisation.  The library never aborts, exits or prints.
 * Numerics: bf16 inputs are multiplied on bf16 matrix cores with fp32
 * accumulation.  The fp32 state enters Q_c S_c, and the masked scores
 * P = tril(Q_c K_c^T) enter P V, each as a sum of two bf16 parts (high and
 * low): about 16 significant bits, a relative error of at most 2^-16.  So
 * integer-valued inputs give exact results as long as every score
 * |q_t . k_s| and every state entry is at most 2^16 in magnitude and every
 * other partial sum (of P V, Q S, K^T V and O) stays below 2^24; one bf16
 * value alone would hold integers exactly only up to 256.  The decode
 * kernels (and the short-prompt route's fused decode steps) run fp32 FMAs:
 * exact while partial sums stay below 2^24; the short-prompt route's chunk
 * on the matrix cores (grouped heads, T >= 8) has the bounds above.  fp32 inputs use fp32 matrix-core instructions
 * throughout, exact under the same 2^24 condition.  FP8 inputs (the 8-bit format
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
    LLA_ERR_UNSUPPORTED = 4, /* unknown option bits */
    LLA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned (a gate: 4-byte) */
    LLA_ERR_ALIAS = 6,       /* an output overlaps an input, another output or the workspace */
    LLA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than lla_prefill_workspace_size() */
    LLA_ERR_DEVICE = 8,      /* a HIP call failed (see lla_last_device_error) */
    LLA_ERR_SCRATCH = 9      /* lla_prefill_noalloc: the shape needs more workspace than
                                LLA_NOALLOC_SCRATCH_BYTES */
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
 * Number G of consecutive chunks of c tokens (c = C, or ceil(C/2) for
 * C > 64) one workgroup walks in lla_prefill (a "segment"); a sequence has
 * ceil(ceil(T/c) / G) segments.  The choice
 * depends on the shape only (not on the device), so results are
 * reproducible across devices.  Returns 0 for invalid sizes.
 */
int64_t lla_prefill_segment_chunks(int64_t B, int64_t H, int64_t T, int64_t dk,
                                   int64_t dv, int64_t C);

/*
 * Bytes of device workspace for this shape: one fp32 dk x dv state per
 * segment per (b, h) when a sequence has more than one segment, else 0 --
 * what lla_prefill requires -- or more for a shape that can run as one launch
 * (see lla_prefill_ex): room for that route's published segment sums.  A call
 * given only the states' size still runs that route, with the same results,
 * without publishing.  Returns 0 for invalid sizes as well.
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
 *    fp32 -- holds S after s*G*c tokens (G = lla_prefill_segment_chunks, c as
 *    above; for an even C, G*c is a whole number of chunks of C).
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
 * T * G <= 64) the state is read and written once for all T tokens.  With
 * one query head per state, or fp32 inputs, the call runs T fused decode
 * steps (the state held in registers between the steps) with the arithmetic
 * of lla_decode_step (lla_decode_step_gqa), so its results equal T
 * successive decode-step calls bit for bit.  With several query heads per
 * state, bf16 or FP8 inputs and T >= 8 it runs the T tokens' G query heads
 * as one chunk on the matrix cores (the numerics of the chunked prefill
 * above: integers exact within its bounds, floats within its error, not the
 * bits of decode steps); with T < 8 the fused decode steps are used there
 * too.  The workspace is not touched on this route (it is still validated).
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
 * T * G <= 64 take the short-prompt route described at lla_prefill.
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
 *   LLA_PREFILL_KEEP_STATE: S is read but not written -- the verify pass of
 *     speculative decoding (blog "A 128 000 tokens, l'attention avale 85 % du
 *     calcul", on speculative decoding adding tokens per decode iteration):
 *     the T draft tokens' outputs o_1..o_T are computed from S_0 and S keeps
 *     S_0, so that lla_state_commit can then advance it by the accepted
 *     prefix only.  On the fused short-prompt route (1 <= T <= 16,
 *     dk = dv in {64, 128}, T * G <= 64 with shared-state heads) o_t equals
 *     what t decode steps give, bit for bit; other shapes take the chunked
 *     path, whose outputs are those of the same call without the option
 *     (the prefill's numerics).  With LLA_PREFILL_ZERO_STATE too, S is neither
 *     read nor written; with T = 0 nothing is written.
 */
#define LLA_PREFILL_KEEP_STATE 2u

/*
 * lla_prefill_gqa with options (a bitwise OR of LLA_PREFILL_* values, 0 for
 * none); unknown bits give LLA_ERR_UNSUPPORTED.  With flags = 0 and Hq = Hkv
 * this is lla_prefill; the workspace is that of lla_prefill_gqa_workspace_size.
 * Results with LLA_PREFILL_ZERO_STATE equal those of lla_state_init followed
 * by the call without it, bit for bit.
 *
 * With either option S is not both read and written, and a shape with
 * several segments but at most 16 chunks (of c tokens) before its last
 * segment -- bf16 or FP8 inputs, head dims up to 64 (or rows that are not
 * whole 16-byte vectors) -- runs as one kernel: every segment's walk sums the
 * earlier segments' K^T V itself, in the order of the segment pass and the
 * scan, so the results are the bits of the three phases.  Given the
 * workspace lla_prefill_gqa_workspace_size reports, every segment but the
 * last first sums its own chunks and publishes the sum there, and a later
 * segment's walk reads a published sum instead of summing that segment
 * again (when both workgroups run on one XCD and the sum arrives within a
 * short bounded wait; otherwise it sums it itself -- the same bits either
 * way).  A call enqueued while its stream is capturing a HIP graph does not
 * publish: a flag value unique to each call tells this call's sums from an
 * earlier call's, and a graph would replay one value.  The workspace's
 * content on return is unspecified on this route.
 */
/*
 * How long, in ticks of the GPU's 100 MHz real-time counter, a walk on the
 * one-launch route waits for an earlier segment's published sum before it
 * sums that segment itself (default 2000, 20 us), for the calls enqueued
 * after this one in the process.  Results never depend on it: any segment
 * not yet published when the wait ends is summed with the same products in
 * the same order.  0 polls each flag once.  For tests of that fallback and
 * for tuning; LLA_ERR_SHAPE for a negative value.
 */
lla_status lla_set_publish_wait_ticks(int64_t ticks);

lla_status lla_prefill_ex(const void *Q, const void *K, const void *V, lla_dtype dtype,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk,
                          int64_t dv, int64_t C, unsigned flags, float *S, float *O,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * The commit after a verify pass (LLA_PREFILL_KEEP_STATE): for every
 * sequence b and key/value head h,
 *     S[b][h] += sum over t < m_b of k_t v_t^T,
 * where m_b = accepted[b] is the number of draft tokens sequence b accepted
 * (clamped to [0, T]; NULL means all T).  Each state element receives one
 * fmaf per token in token order -- the update lla_decode_step applies -- so
 * after the commit S equals the state m_b decode steps would leave, bit for
 * bit; a sequence with m_b = 0 is neither read nor written.  K, V: the draft
 * tokens as given to the verify pass, [B][H][T][dk] and [B][H][T][dv]
 * (dtype), H = key/value heads; accepted: device array of B int32 (read on
 * the device: the acceptance decision never has to reach the host); S:
 * [B][H][dk][dv] fp32, in place.  Limits and errors as lla_prefill (no chunk
 * size); T = 0 is a no-op.
 */
lla_status lla_state_commit(const void *K, const void *V, lla_dtype dtype, int64_t B, int64_t H,
                            int64_t T, int64_t dk, int64_t dv, const int32_t *accepted, float *S,
                            void *stream);

/*
 * lla_prefill_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call itself allocates nothing and
 * calls no allocating routine.  The workspace lla_prefill_ex would take
 * (lla_prefill_gqa_workspace_size bytes) is a static device array of
 * LLA_NOALLOC_SCRATCH_BYTES inside the library, one per device, held from the
 * first call on that device until the process ends; that first call looks up
 * its address (hipGetSymbolAddress, with the stream's device made current for
 * the lookup).  The stream's device is the one used (the current device for
 * the NULL stream).
 *
 * Every call on a device shares that device's array, and it keeps the last
 * call's contents: nothing in it needs to start at zero (each call writes
 * every state it reads).  Calls that overlap in time on one device -- on two
 * streams, or from two host threads -- race on the array; serialise them.
 * A graph that captures this call keeps the array's address.
 *
 * Errors as lla_prefill_ex; a shape whose workspace exceeds
 * LLA_NOALLOC_SCRATCH_BYTES (for example more than 512 key/value heads x
 * segments at d_k = d_v = 128) returns LLA_ERR_SCRATCH before any HIP call.
 * Results equal those of lla_prefill_ex on the same arguments bit for bit.
 */
#define LLA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

lla_status lla_prefill_noalloc(const void *Q, const void *K, const void *V, lla_dtype dtype,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk,
                               int64_t dv, int64_t C, unsigned flags, float *S, float *O,
                               void *stream);

/*
 * One decode step with shared-state heads: q: [B][Hq][dk], k: [B][Hkv][dk],
 * v: [B][Hkv][dv] (dtype); S: [B][Hkv][dk][dv] fp32 updated once in place;
 * o: [B][Hq][dv] fp32.  Each state is read from memory once for the G query
 * heads of its group (any G = Hq / Hkv; G = 1 is lla_decode_step).  Per query
 * head the arithmetic is that of lla_decode_step (identical bits).
 */
lla_status lla_decode_step_gqa(const void *q, const void *k, const void *v, lla_dtype dtype,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t dk, int64_t dv,
                               float *S, float *o, void *stream);

/*
 * Gated (decayed) state.  The slide deck "Chunking, causality, and parallel
 * prefill" ("Boundary, evidence, and sources") cites the chunkwise form of
 * gated linear attention but gives no gate; these calls take the plainest
 * decay, one scalar gate g_t per (b,h) and token applied to the previous
 * state before the token's update:
 *     S_t = g_t S_{t-1} + k_t v_t^T,    o_t = S_t^T q_t.
 * With g = 1 this is lla_prefill's recurrence.  gate: fp32, [B][H][T] for
 * the prefill, [B][H] for the decode step, 4-byte aligned, read only.  Gates
 * are taken in [2^-126, 1]: g <= 0 (and NaN) act as 2^-126, g > 1 as 1.
 * One query head per state here; the _gqa forms below take shared-state
 * heads.  Sizes, dtypes, chunk
 * sizes, S, O and the errors are those of lla_prefill; options as
 * lla_prefill_ex: LLA_PREFILL_ZERO_STATE, and LLA_PREFILL_KEEP_STATE for the
 * verify pass of speculative decoding (S not written; then
 * lla_state_commit_gated).  Every prompt length
 * takes the chunked path (segment pass, scan, walk), with the chunked
 * prefill's numerics: the decays scale the masked scores before their bf16
 * high + low split, Q_c S_c is added scaled in fp32, and the state hop takes
 * V scaled as a high + low pair, so results are within the same error of the
 * exact recurrence (integers exact under the same bounds when every gate is 1).
 * The workspace (lla_prefill_gated_workspace_size bytes, 16-byte aligned;
 * 0 with a single segment, then it may be NULL) holds the segment states and
 * one decay per segment; it must not overlap any other buffer.
 */
size_t lla_prefill_gated_workspace_size(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                        int64_t C);

lla_status lla_prefill_gated(const void *Q, const void *K, const void *V, const float *gate,
                             lla_dtype dtype, int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                             int64_t C, unsigned flags, float *S, float *O, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * One gated decode step: S = g S + k v^T, then o = S^T q, for B*H states
 * (gate [B][H]).  Arguments and errors as lla_decode_step.  The arithmetic is
 * lla_decode_step's after the state is scaled by g, so g = 1 gives identical
 * bits.
 */
lla_status lla_decode_step_gated(const void *q, const void *k, const void *v, const float *gate,
                                 lla_dtype dtype, int64_t B, int64_t H, int64_t dk, int64_t dv,
                                 float *S, float *o, void *stream);

/*
 * The gated calls with shared-state heads (as lla_prefill_gqa and
 * lla_decode_step_gqa): Hq query heads read Hkv decayed states, query head h
 * the state h / (Hq / Hkv).  The gates belong to the states: gate
 * [B][Hkv][T] for the prefill, [B][Hkv] for the decode step.  Q, O: Hq
 * heads; K, V, S: Hkv heads.  The workspace is that of
 * lla_prefill_gated_gqa_workspace_size (with several query heads per state it
 * holds the start states even for one segment).  With Hq = Hkv these are the
 * calls above.  lla_state_commit_gated takes the Hkv states and their gates.
 */
size_t lla_prefill_gated_gqa_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk,
                                            int64_t dv, int64_t C);

lla_status lla_prefill_gated_gqa(const void *Q, const void *K, const void *V, const float *gate,
                                 lla_dtype dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t dk,
                                 int64_t dv, int64_t C, unsigned flags, float *S, float *O, void *workspace,
                                 size_t workspace_bytes, void *stream);

lla_status lla_decode_step_gated_gqa(const void *q, const void *k, const void *v, const float *gate,
                                     lla_dtype dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t dk,
                                     int64_t dv, float *S, float *o, void *stream);

/*
 * The commit after a gated verify pass (lla_prefill_gated with
 * LLA_PREFILL_KEEP_STATE): for every sequence b and head h, for the first
 * m_b draft tokens t in order,
 *     S[b][h] <- g_t S[b][h] + k_t v_t^T,
 * with the gated decode step's per-element arithmetic (the decay, then one
 * fmaf), so S equals the state of m_b gated decode steps bit for bit.  gate:
 * the verify pass's [B][H][T] gates (4-byte aligned, read only); the other
 * arguments, limits and errors as lla_state_commit (H states per sequence:
 * with shared-state heads, the Hkv states and their gates).  For callers with
 * a decayed state that
 * speculate (blog "A 128 000 tokens, l'attention avale 85 % du calcul", on
 * speculative decoding adding tokens per decode iteration).
 */
lla_status lla_state_commit_gated(const void *K, const void *V, const float *gate, lla_dtype dtype,
                                  int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                  const int32_t *accepted, float *S, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H */
