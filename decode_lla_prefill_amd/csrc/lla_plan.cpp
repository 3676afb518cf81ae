// lla_plan.cpp -- the prefill plan: how a shape is cut into work for the
// kernels.  Host code only (no kernels): the chunk tile and head-dim tile a
// shape compiles to, the number of chunks one workgroup walks (a segment) and
// whether the walks start from the workspace.  Chunk tiles are 32 or 64 rows.
//
// The chunk form of the slide deck "Chunking, causality, and parallel
// prefill" ("Split into chunks", "Incoming and outgoing state") serialises
// only the chunk-to-chunk state hop.  A sequence of n_c chunks is cut into
// segments of G chunks: each segment's K^T V is summed in parallel, a scan
// over segments gives every segment its starting state, and one workgroup
// walks each segment's chunks.  G depends on the shape alone, never on the
// device, so the rounding order and hence the results are reproducible.
#include "lla_internal.h"

namespace lla {

// Padded tile size (32, 64 or 128) for a head dim or a chunk size.
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
    const int64_t want = p.n_c * p.BHq;  // lines if every segment were one chunk
    p.G = want > kTargetWalkers ? (want + kTargetWalkers - 1) / kTargetWalkers : 1;
    if (p.G > p.n_c) p.G = p.n_c > 0 ? p.n_c : 1;
    p.n_seg = p.n_c > 0 ? (p.n_c + p.G - 1) / p.G : 0;
    // Chunks of more than 64 tokens run as two sub-chunks of ceil(C/2)
    // tokens each, twice as many per segment: the chunk form gives the same
    // result for any chunk size, up to rounding, and the 64-row tiles of the
    // double-buffered walks were measured faster than 128-row ones (fp32
    // tiles of 128 rows would not fit the LDS at all).  For an even C the
    // segments then start at the same tokens as in the plan for C; for an
    // odd C there are never more of them.
    if (p.C > 64 && p.n_c > 0) {
        p.C = (p.C + 1) / 2;
        p.CT = pad_dim(p.C);
        p.n_c = (p.T + p.C - 1) / p.C;
        p.G = 2 * p.G < p.n_c ? 2 * p.G : p.n_c;
        p.n_seg = (p.n_c + p.G - 1) / p.G;
    }
    // a walk reads its starting state from the workspace when there are
    // several segments, or several query heads per state (the group's walks
    // must not read S while one of them writes S_T)
    p.use_ws = p.n_seg > 1 || p.group > 1;
    const int ve = p.dtype == LLA_FP8_E4M3 ? 16 : (p.dtype == LLA_BF16 ? 8 : 4);  // per 16 bytes
    p.vec = (p.dk % ve == 0) && (p.dv % ve == 0);
    p.prefix = false;
    p.publish = false;
    p.token = 0;
    p.wait_ticks = 0;
}

// Whether the shape runs as one launch: few chunks before the last segment
// (each walk can sum them itself), or -- when the earlier segments' sums are
// published -- a few more segments with every XCD's range of workgroup ids
// (xcd_major) holding whole key/value heads, so that every reader finds its
// writers on its own XCD.
static bool prefix_shape(const PrefillPlan& p, bool published) {
    if (p.n_seg <= 1) return false;
    const int64_t before = (p.n_seg - 1) * p.G;
    if (before <= kPrefixMaxChunks) return true;
    if (!published || p.n_seg > kPublishMaxSegments || before > kPublishMaxChunks || p.G > kPublishMaxG)
        return false;
    const int64_t units = p.BHq * p.n_seg * p.n_vb, per_head = (int64_t)p.group * p.n_seg * p.n_vb;
    return units % 8 == 0 && (units / 8) % per_head == 0;
}

bool prefix_capable(const PrefillPlan& p) { return prefix_shape(p, true); }

bool prefix_walk_fits(const PrefillPlan& p, bool published) {
    // bf16 or FP8 on the four-wave walk (d = 128 in whole vectors takes the eight-wave walk)
    if (p.dtype == LLA_F32 || (p.D == 128 && p.vec)) return false;
    return (p.zero_start || p.keep) && prefix_shape(p, published);
}

int64_t prefix_slot_floats(const PrefillPlan& p) { return p.BH * p.n_seg * p.n_vb * 64 * (int64_t)p.D; }

size_t prefix_publish_bytes(const PrefillPlan& p) {
    return (size_t)prefix_slot_floats(p) * sizeof(float) + (size_t)(p.BH * p.n_seg * p.n_vb) * 8u;
}

}  // namespace lla
