// plan.cpp -- host planner for the fused AdamW launch (no HIP calls).
//
// The list's elements are numbered by their position in the flat concatenation
// of the tensors in list order.  One data-parallel rank owns the positions
// [shard_begin, shard_end) (ZeRO optimizer-state sharding as in "Distributed
// optimizer support for BERT"); a tensor that straddles an edge contributes
// only its elements inside the range.  Each contributing piece becomes a
// segment; each segment is cut into workgroup chunks:
//
//   [head: element chunk] [body: vector chunks, 16-byte aligned in every stream] [tail: element chunk]
//
// The head is the smallest count h < 8 that brings every stream's address to a
// 16-byte boundary at the same element; if no such h exists (streams misaligned
// relative to each other), or no whole 8-element pack follows it, the whole
// segment is cut into element chunks.
#include "plan.hpp"

#include <stdio.h>

namespace adamw {

void mode_esizes(adamw_mode mode, adamw_dtype p_dtype, bool for_check, int esz[kStreams])
{
    (void)p_dtype;
    for (int s = 0; s < kStreams; ++s) esz[s] = 0;
    esz[ADAMW_STREAM_GRAD] = 2;
    if (for_check) return;
    esz[ADAMW_STREAM_PARAM] = 2;
    const int state = mode == ADAMW_PURE_KAHAN ? 2 : 4;
    esz[ADAMW_STREAM_EXP_AVG] = state;
    esz[ADAMW_STREAM_EXP_AVG_SQ] = state;
    esz[ADAMW_STREAM_AUX] = mode == ADAMW_MIXED ? 4 : 2;
}

adamw_status check_mode(adamw_mode mode, adamw_dtype p_dtype, bool for_check, std::string& err)
{
    if (for_check) {
        if (p_dtype != ADAMW_F16 && p_dtype != ADAMW_BF16) {
            err = "adamw_check_finite: g_dtype must be ADAMW_F16 or ADAMW_BF16";
            return ADAMW_E_UNSUPPORTED;
        }
        return ADAMW_OK;
    }
    if (mode == ADAMW_MIXED) {
        if (p_dtype != ADAMW_BF16 && p_dtype != ADAMW_F16) {
            err = "ADAMW_MIXED needs p_dtype ADAMW_BF16 or ADAMW_F16";
            return ADAMW_E_UNSUPPORTED;
        }
        return ADAMW_OK;
    }
    if (mode == ADAMW_PURE_KAHAN || mode == ADAMW_MIXED_SPLIT) {
        if (p_dtype != ADAMW_BF16) {
            err = mode == ADAMW_PURE_KAHAN ? "ADAMW_PURE_KAHAN needs p_dtype ADAMW_BF16"
                                           : "ADAMW_MIXED_SPLIT needs p_dtype ADAMW_BF16";
            return ADAMW_E_UNSUPPORTED;
        }
        return ADAMW_OK;
    }
    err = "unknown adamw_mode";
    return ADAMW_E_UNSUPPORTED;
}

static const char* kStreamName[kStreams] = {"param", "grad", "exp_avg", "exp_avg_sq", "aux"};

// Appends the chunks of `count` elements from `off` (at most `per` each) to the
// plan when `build`, and counts them in `n_chunks` either way.
static void push_chunks(Plan& p, bool build, int64_t& n_chunks, uint32_t seg, int64_t off, int64_t count, int64_t per,
                        bool vec)
{
    n_chunks += (count + per - 1) / per;
    if (!build) return;
    while (count > 0) {
        int64_t n = count < per ? count : per;
        DevChunk c;
        c.seg = seg;
        c.n_kind = (uint32_t)n | (vec ? kVecBit : 0u);
        c.off = (uint64_t)off;
        p.chunks.push_back(c);
        off += n;
        count -= n;
    }
}

adamw_status build_plan(const int esz_in[kStreams], const adamw_tensor_list* list, int64_t chunk_elems,
                        int64_t max_chunks, Plan* outp, std::string& err)
{
    char buf[256];
    Plan scratch;
    Plan& out = outp ? *outp : scratch;   // validation only when outp is null
    out = Plan();
    const bool build = outp != nullptr;
    if (!list) { err = "tensor list is null"; return ADAMW_E_INVALID; }
    const int64_t nt = list->n_tensors;
    if (nt < 0) { err = "n_tensors < 0"; return ADAMW_E_INVALID; }
    if (nt > 0 && !list->numel) { err = "numel array is null"; return ADAMW_E_INVALID; }
    if (list->flat_mask & ~(0x1fu | ADAMW_BLOCKED_STATE | ADAMW_FLAT_PAD8)) {
        err = "flat_mask has unknown bits";
        return ADAMW_E_INVALID;
    }
    // the padded flat index: every tensor starts at a multiple of 8
    const int64_t flat_align = (list->flat_mask & ADAMW_FLAT_PAD8) ? 8 : 1;
    // the blocked layout concerns the state streams only: a plan that reads
    // none of them (the overflow check) ignores it
    const bool blocked = (list->flat_mask & ADAMW_BLOCKED_STATE) != 0 &&
                         (esz_in[ADAMW_STREAM_EXP_AVG] || esz_in[ADAMW_STREAM_EXP_AVG_SQ] || esz_in[ADAMW_STREAM_AUX]);

    int64_t total = 0;
    for (int64_t i = 0; i < nt; ++i) {
        int64_t n = list->numel[i];
        if (n < 0) {
            snprintf(buf, sizeof buf, "numel[%lld] = %lld < 0", (long long)i, (long long)n);
            err = buf;
            return ADAMW_E_INVALID;
        }
        if (n > (INT64_C(1) << 56) || total > (INT64_C(1) << 56)) { err = "list too large"; return ADAMW_E_INVALID; }
        total += (n + flat_align - 1) / flat_align * flat_align;
    }
    const int64_t b = list->shard_begin;
    const int64_t e = list->shard_end < 0 ? total : list->shard_end;
    if (list->shard_end < -1 || b < 0 || b > e || e > total) {
        snprintf(buf, sizeof buf, "shard range [%lld, %lld) outside [0, %lld]", (long long)b,
                 (long long)list->shard_end, (long long)total);
        err = buf;
        return ADAMW_E_INVALID;
    }

    int esz[kStreams];
    bool flat[kStreams];
    // blocked state: exp_avg, exp_avg_sq and aux share one flat buffer of the
    // shard in blocks of state_block elements, [exp_avg][exp_avg_sq][aux] each
    int64_t soff[kStreams] = {0, 0, 0, 0, 0}, block_bytes = 0, state_block = 1;
    uintptr_t state_base = 0;
    if (blocked) {
        state_block = kStateBlockElems;
        int64_t acc = 0;
        for (int s = ADAMW_STREAM_EXP_AVG; s <= ADAMW_STREAM_AUX; ++s) {
            soff[s] = acc;
            acc += state_block * esz_in[s];
        }
        block_bytes = acc;
        if (e > b) {
            if (!list->ptr[ADAMW_STREAM_EXP_AVG] || !list->ptr[ADAMW_STREAM_EXP_AVG][0] ||
                (uintptr_t)list->ptr[ADAMW_STREAM_EXP_AVG][0] % 16u) {
                err = "blocked state buffer (ptr[2][0]) is null or not 16-byte aligned";
                return ADAMW_E_INVALID;
            }
            state_base = (uintptr_t)list->ptr[ADAMW_STREAM_EXP_AVG][0];
        }
    }
    for (int s = 0; s < kStreams; ++s) {
        esz[s] = esz_in[s];
        flat[s] = (list->flat_mask >> s) & 1u;
        if (!esz[s]) continue;
        if (blocked && s >= ADAMW_STREAM_EXP_AVG) continue;
        bool needed = flat[s] ? (e > b) : (nt > 0);
        if (needed && !list->ptr[s]) {
            snprintf(buf, sizeof buf, "pointer array of stream %s is null", kStreamName[s]);
            err = buf;
            return ADAMW_E_INVALID;
        }
        if (flat[s] && e > b) {
            uintptr_t a = (uintptr_t)list->ptr[s][0];
            if (!a || a % (uintptr_t)esz[s]) {
                snprintf(buf, sizeof buf, "flat %s buffer is null or not %d-byte aligned", kStreamName[s], esz[s]);
                err = buf;
                return ADAMW_E_INVALID;
            }
        }
    }
    if (chunk_elems < 2048 || chunk_elems % 2048) { err = "bad chunk size"; return ADAMW_E_INVALID; }

    int64_t base = 0, nseg = 0, n_chunks = 0;
    for (int64_t i = 0; i < nt; ++i) {
        const int64_t n = list->numel[i];
        const int64_t lo = b > base ? b : base;
        const int64_t hi = e < base + n ? e : base + n;
        // a blocked state splits the piece at block boundaries (relative to b)
        for (int64_t plo = lo; plo < hi;) {
            int64_t phi = hi;
            if (blocked) {
                const int64_t next = b + ((plo - b) / state_block + 1) * state_block;
                if (next < phi) phi = next;
            }
            SegInfo si{i, plo - base, plo, phi - plo};
            DevSeg d{};
            for (int s = 0; s < kStreams; ++s) {
                if (!esz[s]) continue;
                uintptr_t a;
                if (blocked && s >= ADAMW_STREAM_EXP_AVG) {
                    const int64_t rel = plo - b;
                    a = state_base + (uintptr_t)((rel / state_block) * block_bytes + soff[s] +
                                                 (rel % state_block) * esz[s]);
                } else if (flat[s]) {
                    a = (uintptr_t)list->ptr[s][0] + (uintptr_t)((plo - b) * esz[s]);
                } else {
                    uintptr_t t0 = (uintptr_t)list->ptr[s][i];
                    if (!t0 || t0 % (uintptr_t)esz[s]) {
                        snprintf(buf, sizeof buf, "%s pointer of tensor %lld is null or not %d-byte aligned",
                                 kStreamName[s], (long long)i, esz[s]);
                        err = buf;
                        return ADAMW_E_INVALID;
                    }
                    a = t0 + (uintptr_t)((plo - base) * esz[s]);
                }
                d.ptr[s] = (uint64_t)a;
            }
            plo = phi;
            if (nseg >= (int64_t)UINT32_MAX) { err = "too many segments"; return ADAMW_E_INVALID; }
            const uint32_t seg = (uint32_t)nseg++;
            if (build) {
                out.segs.push_back(d);
                out.info.push_back(si);
            }

            // head peel: smallest h in [0, 8) aligning every active stream to 16 bytes
            int head = -1;
            for (int h = 0; h < kPack && head < 0; ++h) {
                bool ok = true;
                for (int s = 0; s < kStreams && ok; ++s)
                    if (esz[s]) ok = ((d.ptr[s] + (uint64_t)h * esz[s]) % 16u) == 0;
                if (ok) head = h;
            }
            const int64_t cnt = si.count;
            // no full pack after the head: one element pass over the piece
            if (head < 0 || cnt - head < kPack) {
                push_chunks(out, build, n_chunks, seg, 0, cnt, kElemChunkElems, false);
            } else {
                const int64_t body = (cnt - head) / kPack * kPack;
                push_chunks(out, build, n_chunks, seg, 0, head, kElemChunkElems, false);
                push_chunks(out, build, n_chunks, seg, head, body, chunk_elems, true);
                push_chunks(out, build, n_chunks, seg, head + body, cnt - head - body, kElemChunkElems, false);
            }
            if (n_chunks > max_chunks) {
                snprintf(buf, sizeof buf,
                         "more than %lld chunks in one launch (a grid holds at most 2^32 - 1 lanes): "
                         "split the list or raise the chunk size",
                         (long long)max_chunks);
                err = buf;
                return ADAMW_E_INVALID;
            }
        }
        base += (n + flat_align - 1) / flat_align * flat_align;
    }
    out.total = e - b;
    return ADAMW_OK;
}

void chunk_bytes(const Plan& plan, size_t c, const int esz[kStreams], uint64_t lo[kStreams], uint64_t hi[kStreams])
{
    const DevChunk& ch = plan.chunks[c];
    const DevSeg& sg = plan.segs[ch.seg];
    const uint64_t n = ch.n_kind & kCountMask;
    for (int s = 0; s < kStreams; ++s) {
        if (!esz[s]) {
            lo[s] = hi[s] = 0;
            continue;
        }
        lo[s] = sg.ptr[s] + ch.off * (uint64_t)esz[s];
        hi[s] = lo[s] + n * (uint64_t)esz[s];
    }
}

adamw_status build_copy_plan(const int esz_in[kStreams], const adamw_tensor_list* list, uint64_t blocked,
                             CopyPlan* out, std::string& err)
{
    if (!list) { err = "tensor list is null"; return ADAMW_E_INVALID; }
    if (list->flat_mask & ADAMW_BLOCKED_STATE) {
        err = "the list describes the per-tensor state: leave ADAMW_BLOCKED_STATE out of its flat_mask "
              "(the blocked buffer is its own argument)";
        return ADAMW_E_INVALID;
    }
    int esz[kStreams] = {0, 0, esz_in[2], esz_in[3], esz_in[4]};
    // the per-tensor side: pointers, alignment, shard range
    adamw_status st = build_plan(esz, list, kStateBlockElems, kMaxCopyChunks, nullptr, err);
    if (st != ADAMW_OK) return st;
    // the blocked side: the pieces of the blocked plan and their addresses there
    void* const blocked_ptr[1] = {reinterpret_cast<void*>((uintptr_t)blocked)};
    adamw_tensor_list bl = *list;
    bl.flat_mask |= ADAMW_BLOCKED_STATE;
    bl.ptr[ADAMW_STREAM_EXP_AVG] = blocked_ptr;
    Plan plan;
    st = build_plan(esz, &bl, kStateBlockElems, kMaxCopyChunks, &plan, err);
    if (st != ADAMW_OK) return st;
    out->segs.resize(plan.segs.size());
    for (size_t i = 0; i < plan.segs.size(); ++i) {
        const SegInfo& si = plan.info[i];
        DevCopySeg& c = out->segs[i];
        c = DevCopySeg{};
        for (int s = ADAMW_STREAM_EXP_AVG; s <= ADAMW_STREAM_AUX; ++s) {
            if (!esz[s]) continue;
            const uint64_t e = (uint64_t)esz[s];
            c.blocked_side[s - 2] = plan.segs[i].ptr[s];
            if ((list->flat_mask >> s) & 1u)
                c.tensor_side[s - 2] = (uint64_t)(uintptr_t)list->ptr[s][0] + (uint64_t)(si.flat - list->shard_begin) * e;
            else
                c.tensor_side[s - 2] = (uint64_t)(uintptr_t)list->ptr[s][si.tensor] + (uint64_t)si.tensor_off * e;
        }
    }
    out->chunks.swap(plan.chunks);
    int64_t block_bytes = 0;
    for (int s = ADAMW_STREAM_EXP_AVG; s <= ADAMW_STREAM_AUX; ++s) block_bytes += kStateBlockElems * esz[s];
    out->blocked_bytes = (plan.total + kStateBlockElems - 1) / kStateBlockElems * block_bytes;
    return ADAMW_OK;
}

size_t choose_plan_slot(const std::vector<bool>& pinned, size_t cap)
{
    size_t unpinned = 0, lru = pinned.size();
    for (size_t i = 0; i < pinned.size(); ++i) {
        if (pinned[i]) continue;
        ++unpinned;
        lru = i;   // the last unpinned slot in MRU order
    }
    return unpinned < cap ? pinned.size() : lru;
}

void plan_key(int64_t tag, const int esz[kStreams], const adamw_tensor_list* list, int64_t chunk_elems,
              std::vector<int64_t>& key)
{
    const int64_t nt = list->n_tensors;
    key.clear();
    key.reserve(12 + (size_t)nt * 6);
    key.push_back(tag);
    for (int s = 0; s < kStreams; ++s) key.push_back(esz[s]);
    key.push_back(chunk_elems);
    key.push_back(nt);
    key.push_back(list->shard_begin);
    key.push_back(list->shard_end);
    key.push_back((int64_t)list->flat_mask);
    for (int64_t i = 0; i < nt; ++i) key.push_back(list->numel[i]);
    const bool blocked = (list->flat_mask & ADAMW_BLOCKED_STATE) != 0;
    for (int s = 0; s < kStreams; ++s) {
        if (!esz[s] || !list->ptr[s] || (blocked && s > ADAMW_STREAM_EXP_AVG)) {
            key.push_back(-1);
            continue;
        }
        if (((list->flat_mask >> s) & 1u) || (blocked && s == ADAMW_STREAM_EXP_AVG)) {
            key.push_back((int64_t)(uintptr_t)list->ptr[s][0]);
        } else {
            for (int64_t i = 0; i < nt; ++i) key.push_back((int64_t)(uintptr_t)list->ptr[s][i]);
        }
    }
}

}  // namespace adamw
