// Work plans of the chunked prefill and of the backward pass: host arithmetic
// only (no HIP call), so that it builds and is tested on its own, with or
// without a device.
#include <algorithm>

#include "kda_internal.hpp"

namespace kda {

PrefillPlan plan_prefill_scan(bool packed, int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                              int n_cu, int64_t forced, int tier)
{
    constexpr int64_t CH = kChunk;
    PrefillPlan p;
    p.tier = 2;
    if (n_seq <= 0 || H <= 0 || tier >= 2 || n_cu <= 0) return p;
    const int64_t rows = packed ? T_total : n_seq * T;
    int64_t seg = forced;
    if (seg <= 0) {
        const int64_t per_cu = (rows * H + n_cu - 1) / n_cu;
        seg = std::max<int64_t>(kMinSegment, (per_cu + CH - 1) / CH * CH);
    }
    // T/P blocks: one per (chunk id, head), ids below rows / 64 + sequences + 1
    const int64_t tp_ids = rows / CH + n_seq + 1;
    const bool tp_ok = tier == 0 && static_cast<double>(tp_ids) * H * kTpBytes <= kTpCap;
    int64_t seg0 = seg, seg_min = seg, nseg_dense = 1, n_segs = 0, slots = 0;
    bool tp = false;
    size_t plan_bytes = 0;
    if (!packed) {
        auto dense_segments = [&](int64_t s0, int64_t s) {
            return T > s0 ? 1 + (T - s0 + s - 1) / s : int64_t(1);
        };
        int64_t seg_tp = seg, seg0_tp = seg;
        if (forced <= 0 && T > seg) {
            const int64_t k = (T + seg - 1) / seg;  // segments at the plain length
            // T = k L + (3/5) L
            const int64_t even = (5 * T + 5 * k + 2) / (5 * k + 3);
            seg_tp = std::max<int64_t>(kMinSegment, (even + CH - 1) / CH * CH);
            seg0_tp = seg_tp;
        }
        tp = tp_ok && dense_segments(seg0_tp, seg_tp) > 1;
        if (tp) {
            seg = seg_tp;
            seg0 = seg0_tp;
        } else if (forced <= 0 && T > seg) {
            const int64_t k = (T + seg - 1) / seg;
            const int64_t even = (8 * T + 8 * k + 6) / (8 * k + 7);
            seg = std::max<int64_t>(kMinSegment, (even + CH - 1) / CH * CH);
            seg0 = std::min<int64_t>(seg, (seg * 7 / 8 + CH - 1) / CH * CH);
        }
        nseg_dense = dense_segments(seg0, seg);
        if (nseg_dense < 2) return p;
        n_segs = slots = n_seq * nseg_dense;
        seg_min = seg;
    } else {
        if (forced <= 0) seg_min = std::max<int64_t>(kMinSegment, (seg / 8 + CH - 1) / CH * CH);
        if (T_total <= seg_min) return p;  // no sequence is longer than a segment
        const int64_t per_min = (T_total + seg_min - 1) / seg_min;
        n_segs = n_seq + per_min;
        slots = std::min<int64_t>(n_segs, 2 * per_min);
        // seg_first [n_seq + 2], ws_first [n_seq + 1], seg_order [n_segs]
        plan_bytes = ((2 * static_cast<size_t>(n_seq) + 3 + static_cast<size_t>(n_segs)) * 4 + 255) /
                     256 * 256;
        tp = tp_ok;
    }
    p.tier = tp ? 0 : 1;
    p.segmented = true;
    p.tp = tp;
    p.seg = seg;
    p.seg0 = seg0;
    p.seg_min = seg_min;
    p.nseg_dense = packed ? 0 : nseg_dense;
    p.n_segs = n_segs;
    p.slots = slots;
    p.plan_bytes = plan_bytes;
    p.tp_blocks = tp ? tp_ids : 0;
    p.ws_bytes = plan_bytes + static_cast<size_t>(slots) * H * 3 * kStateFloats * sizeof(float) +
                 static_cast<size_t>(p.tp_blocks) * H * kTpBytes;
    return p;
}

BackwardPlan plan_backward(bool packed, int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                          bool bf16)
{
    BackwardPlan p;
    if (n_seq <= 0 || H <= 0) return p;
    const int64_t rows = packed ? T_total : n_seq * T;
    if (bf16) {
        // chunked: one workspace slot per (chunk id, head); ids below rows / 64 + sequences + 1
        p.chunked = true;
        p.n_ids = rows / kChunk + n_seq + 1;
        p.ws_bytes = static_cast<size_t>(p.n_ids) * H * kChunkBackwardFloats * sizeof(float);
        return p;
    }
    // One checkpoint slot per block of kBackwardBlock tokens: dense, every
    // sequence ceil(T / cb); packed, fewer than T_total / cb + n_seq in all.
    const int64_t cb = kBackwardBlock;
    p.n_slots = rows <= 0 ? 0 : packed ? T_total / cb + n_seq : n_seq * ((T + cb - 1) / cb);
    p.ws_bytes = static_cast<size_t>(p.n_slots) * H * kStateFloats * sizeof(float);
    return p;
}

}  // namespace kda
