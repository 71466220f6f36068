// plan_check.cpp -- the library's host-side logic under AddressSanitizer and
// UndefinedBehaviorSanitizer: the planner, the argument checks and the plan
// cache policy, driven on the CPU with synthetic (never dereferenced) device
// addresses.  Built by tests/test_sanitizers.py with g++ together with
// plan.cpp and validate.cpp; prints "plan_check ok" and a checksum of every
// plan it built (the same with and without the sanitizers), or aborts.
//
// Besides running the code under the sanitizers, every plan built here is
// checked chunk by chunk: each chunk's byte range in every stream lies inside
// the buffer the caller handed in for that stream (inside one block's
// sub-array for the blocked state), vector chunks hold whole 8-element packs
// at 16-byte-aligned addresses, and each segment and chunk index is in range.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "plan.hpp"

using namespace adamw;

namespace {

int g_fail = 0;
uint64_t g_sum = 1469598103934665603ull;

void mix(uint64_t x)
{
    g_sum = (g_sum ^ x) * 1099511628211ull;
}

#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                       \
            if (g_fail > 20) abort();                                       \
        }                                                                   \
    } while (0)

struct Rng {
    uint64_t s;
    uint64_t next()
    {
        s ^= s << 13;
        s ^= s >> 7;
        s ^= s << 17;
        return s;
    }
    int64_t below(int64_t n) { return n > 0 ? (int64_t)(next() % (uint64_t)n) : 0; }
};

// A list as a caller would hand it in, with the buffers' extents remembered.
struct List {
    std::vector<int64_t> numel;
    std::vector<std::vector<void*>> ptr = std::vector<std::vector<void*>>(kStreams);
    int64_t shard_begin = 0, shard_end = -1;
    uint32_t flat_mask = 0;
    adamw_tensor_list c{};

    const adamw_tensor_list* get()
    {
        c.n_tensors = (int64_t)numel.size();
        c.numel = numel.empty() ? nullptr : numel.data();
        for (int s = 0; s < kStreams; ++s) c.ptr[s] = ptr[s].empty() ? nullptr : ptr[s].data();
        c.shard_begin = shard_begin;
        c.shard_end = shard_end;
        c.flat_mask = flat_mask;
        return &c;
    }
};

uint64_t addr(void* p) { return (uint64_t)(uintptr_t)p; }
void* fake(uint64_t a) { return (void*)(uintptr_t)a; }

// Checks every chunk of `plan` against the buffers of `L` (element sizes esz).
void check_chunks(const Plan& plan, List& L, const int esz[kStreams])
{
    const int64_t fa = (L.flat_mask & ADAMW_FLAT_PAD8) ? 8 : 1;
    std::vector<int64_t> start(L.numel.size());
    int64_t total = 0;
    for (size_t i = 0; i < L.numel.size(); ++i) {
        start[i] = total;
        total += (L.numel[i] + fa - 1) / fa * fa;
    }
    const int64_t b = L.shard_begin, e = L.shard_end < 0 ? total : L.shard_end;
    const bool blocked = (L.flat_mask & ADAMW_BLOCKED_STATE) && (esz[2] || esz[3] || esz[4]);
    int64_t soff[kStreams] = {0, 0, 0, 0, 0}, block_bytes = 0;
    for (int s = 2; s < kStreams; ++s) {
        soff[s] = block_bytes;
        block_bytes += kStateBlockElems * esz[s];
    }
    const int64_t nb = (e - b + kStateBlockElems - 1) / kStateBlockElems;
    int64_t covered = 0;
    CHECK(plan.segs.size() == plan.info.size());
    for (size_t c = 0; c < plan.chunks.size(); ++c) {
        const DevChunk& ch = plan.chunks[c];
        CHECK(ch.seg < plan.segs.size());
        if (ch.seg >= plan.segs.size()) continue;
        const SegInfo& si = plan.info[ch.seg];
        const int64_t n = ch.n_kind & kCountMask;
        const bool vec = (ch.n_kind & kVecBit) != 0;
        CHECK(n > 0);
        CHECK(si.tensor >= 0 && si.tensor < (int64_t)L.numel.size());
        CHECK((int64_t)ch.off + n <= si.count);
        covered += n;
        if (vec) CHECK(n % 8 == 0);
        uint64_t lo[kStreams], hi[kStreams];
        chunk_bytes(plan, c, esz, lo, hi);
        const int64_t flat = si.flat + (int64_t)ch.off;
        CHECK(flat >= b && flat + n <= e);
        for (int s = 0; s < kStreams; ++s) {
            mix(lo[s]);
            mix(hi[s]);
            if (!esz[s]) {
                CHECK(lo[s] == 0 && hi[s] == 0);
                continue;
            }
            if (vec) CHECK(lo[s] % 16 == 0);
            uint64_t blo, bhi;   // the buffer (or block sub-array) the range must lie in
            if (blocked && s >= 2) {
                const int64_t rel = flat - b, k = rel / kStateBlockElems;
                CHECK(k < nb);
                blo = addr(L.ptr[2][0]) + (uint64_t)(k * block_bytes + soff[s]);
                bhi = blo + (uint64_t)(kStateBlockElems * esz[s]);
            } else if ((L.flat_mask >> s) & 1u) {
                blo = addr(L.ptr[s][0]);
                bhi = blo + (uint64_t)((e - b) * esz[s]);
            } else {
                blo = addr(L.ptr[s][(size_t)si.tensor]);
                bhi = blo + (uint64_t)(L.numel[(size_t)si.tensor] * esz[s]);
            }
            CHECK(lo[s] >= blo && hi[s] <= bhi && hi[s] - lo[s] == (uint64_t)(n * esz[s]));
        }
    }
    int64_t owned = 0;
    for (size_t i = 0; i < L.numel.size(); ++i) {
        const int64_t lo = start[i] > b ? start[i] : b;
        const int64_t hi = start[i] + L.numel[i] < e ? start[i] + L.numel[i] : e;
        if (hi > lo) owned += hi - lo;
    }
    CHECK(covered == owned);
    CHECK(plan.total == e - b);
}

const int kEszModes[][kStreams] = {
    {2, 2, 4, 4, 4},   // mixed
    {2, 2, 2, 2, 2},   // Kahan
    {2, 2, 4, 4, 2},   // split
    {2, 2, 4, 2, 2},   // pure, fp32 exp_avg
    {2, 2, 2, 4, 0},   // pure, fp32 exp_avg_sq, no compensation
    {0, 2, 0, 0, 0},   // overflow check
};

void random_list(Rng& r, List& L, const int esz[kStreams], bool large)
{
    const int64_t nt = large ? 10000 : r.below(40);
    L.numel.resize((size_t)nt);
    for (auto& n : L.numel) {
        if (large) {
            // log-uniform in [1, 2^22], as the 10,000-tensor fp16 workload
            const double u = (double)(r.next() >> 11) / 9007199254740992.0;
            n = (int64_t)exp(u * log(4194305.0));
            if (n < 1) n = 1;
            if (n > (1 << 22)) n = 1 << 22;
        } else {
            const int64_t k = r.below(3);
            n = k == 0 ? r.below(9) : k == 1 ? 9 + r.below(3000) : 3000 + r.below(70000);
        }
    }
    const bool state = esz[2] || esz[3] || esz[4];
    L.flat_mask = 0;
    if (state && r.below(2)) L.flat_mask |= ADAMW_BLOCKED_STATE;
    if (r.below(2)) L.flat_mask |= ADAMW_FLAT_PAD8;
    const int64_t fa = (L.flat_mask & ADAMW_FLAT_PAD8) ? 8 : 1;
    int64_t total = 0;
    for (int64_t n : L.numel) total += (n + fa - 1) / fa * fa;
    L.shard_begin = 0;
    L.shard_end = -1;
    if (total && r.below(2)) {
        L.shard_begin = r.below(total + 1);
        L.shard_end = L.shard_begin + r.below(total - L.shard_begin + 1);
    }
    const int64_t e = L.shard_end < 0 ? total : L.shard_end;
    for (int s = 0; s < kStreams; ++s) {
        L.ptr[s].clear();
        if (!esz[s]) continue;
        const uint64_t base = ((uint64_t)1 << 40) + ((uint64_t)s << 36) + ((uint64_t)r.below(64) << 21);
        const bool blocked_s = (L.flat_mask & ADAMW_BLOCKED_STATE) && s >= 2;
        if (blocked_s) {
            if (s == 2) L.ptr[s].push_back(fake(((uint64_t)6 << 36) + ((uint64_t)1 << 40) + 256 * r.below(64)));
            continue;
        }
        if (e > L.shard_begin && r.below(3) == 0) {
            L.flat_mask |= 1u << s;
            L.ptr[s].push_back(fake(base + (uint64_t)(esz[s] * r.below(8))));
            continue;
        }
        const int64_t align = r.below(3) == 0 ? 1 : r.below(2) ? 8 : 128;
        uint64_t a = base + (uint64_t)(esz[s] * r.below(8));
        for (int64_t n : L.numel) {
            L.ptr[s].push_back(fake(a));
            a += (uint64_t)(((n + align - 1) / align * align) * esz[s]);
        }
    }
}

void test_random_plans()
{
    Rng r{0x9e3779b97f4a7c15ull};
    for (int it = 0; it < 400; ++it) {
        const int* esz = kEszModes[r.below(6)];
        List L;
        random_list(r, L, esz, it % 100 == 7);
        mix((uint64_t)L.numel.size());
        const bool large = it % 100 == 7;
        const int64_t chunk = large ? 16384 : 2048 * (1 + r.below(8));
        Plan plan;
        std::string err;
        const adamw_status st = build_plan(esz, L.get(), chunk, kMaxUpdateChunks, &plan, err);
        std::string err2;
        CHECK(build_plan(esz, L.get(), chunk, kMaxUpdateChunks, nullptr, err2) == st);
        CHECK(st == ADAMW_OK);
        if (st != ADAMW_OK) {
            fprintf(stderr, "unexpected error: %s\n", err.c_str());
            continue;
        }
        check_chunks(plan, L, esz);
        std::vector<int64_t> key;
        plan_key(3, esz, L.get(), chunk, key);
        for (int64_t k : key) mix((uint64_t)k);
    }
}

// The copy plan between per-tensor state and the blocked buffer: every piece's
// two sides lie inside their buffers (the per-tensor buffer of the piece's
// tensor, or the flat shard buffer; one block's sub-array) and the pieces
// cover the owned elements once.
void test_copy_plans()
{
    Rng r{0x51ed2701a3c4f5e9ull};
    int planned = 0;
    for (int it = 0; it < 300; ++it) {
        const int* esz = kEszModes[r.below(5)];
        List L;
        random_list(r, L, esz, false);
        L.flat_mask &= ~ADAMW_BLOCKED_STATE;
        if (L.ptr[3].empty() && esz[3]) continue;   // random_list gave these streams to a blocked buffer
        const uint64_t blocked = ((uint64_t)7 << 36) + ((uint64_t)1 << 40) + 256 * (uint64_t)r.below(64);
        CopyPlan cp;
        std::string err;
        const adamw_status st = build_copy_plan(esz, L.get(), blocked, &cp, err);
        CHECK(st == ADAMW_OK);
        if (st != ADAMW_OK) {
            fprintf(stderr, "copy plan refused: %s\n", err.c_str());
            continue;
        }
        ++planned;
        const int64_t fa = (L.flat_mask & ADAMW_FLAT_PAD8) ? 8 : 1;
        int64_t total = 0;
        std::vector<int64_t> start;
        for (int64_t n : L.numel) {
            start.push_back(total);
            total += (n + fa - 1) / fa * fa;
        }
        const int64_t b = L.shard_begin, e = L.shard_end < 0 ? total : L.shard_end;
        int64_t block_bytes = 0, soff[3] = {0, 0, 0};
        for (int s = 0; s < 3; ++s) {
            soff[s] = block_bytes;
            block_bytes += kStateBlockElems * esz[s + 2];
        }
        const int64_t nb = (e - b + kStateBlockElems - 1) / kStateBlockElems;
        CHECK(cp.blocked_bytes == nb * block_bytes);
        int64_t covered = 0;
        for (const DevChunk& ch : cp.chunks) {
            CHECK(ch.seg < cp.segs.size());
            const DevCopySeg& sg = cp.segs[ch.seg];
            const uint64_t n = ch.n_kind & kCountMask;
            covered += (int64_t)n;
            for (int s = 0; s < 3; ++s) {
                const int es = esz[s + 2];
                if (!es) {
                    CHECK(sg.tensor_side[s] == 0 && sg.blocked_side[s] == 0);
                    continue;
                }
                // blocked side: inside one block's sub-array for stream s
                const uint64_t lo = sg.blocked_side[s] + ch.off * (uint64_t)es, hi = lo + n * (uint64_t)es;
                CHECK(lo >= blocked && hi <= blocked + (uint64_t)(nb * block_bytes));
                const uint64_t in_block = (lo - blocked) % (uint64_t)block_bytes;
                CHECK(in_block >= (uint64_t)soff[s] && in_block + (hi - lo) <= (uint64_t)(soff[s] + kStateBlockElems * es));
                // tensor side: inside the flat shard buffer, or inside one tensor's buffer
                const uint64_t tlo = sg.tensor_side[s] + ch.off * (uint64_t)es, thi = tlo + n * (uint64_t)es;
                const std::vector<void*>& P = L.ptr[s + 2];
                bool inside = false;
                if ((L.flat_mask >> (s + 2)) & 1u) {
                    inside = tlo >= addr(P[0]) && thi <= addr(P[0]) + (uint64_t)((e - b) * es);
                } else {
                    for (size_t i = 0; i < P.size() && !inside; ++i)
                        inside = tlo >= addr(P[i]) && thi <= addr(P[i]) + (uint64_t)(L.numel[i] * es);
                }
                CHECK(inside);
            }
        }
        int64_t owned = 0;
        for (size_t i = 0; i < L.numel.size(); ++i) {
            const int64_t lo = start[i] > b ? start[i] : b;
            const int64_t hi = start[i] + L.numel[i] < e ? start[i] + L.numel[i] : e;
            if (hi > lo) owned += hi - lo;
        }
        CHECK(covered == owned);
        mix((uint64_t)cp.blocked_bytes);
    }
    CHECK(planned > 100);
}

void expect_invalid(const int esz[kStreams], List& L, const char* what)
{
    Plan plan;
    std::string err;
    const adamw_status st = build_plan(esz, L.get(), 16384, kMaxUpdateChunks, &plan, err);
    CHECK(st != ADAMW_OK);
    CHECK(!err.empty());
    if (st == ADAMW_OK) fprintf(stderr, "accepted: %s\n", what);
}

void test_invalid_lists()
{
    const int* esz = kEszModes[0];
    std::string err;
    Plan plan;
    CHECK(build_plan(esz, nullptr, 16384, kMaxUpdateChunks, &plan, err) == ADAMW_E_INVALID);
    auto base = [&](List& L) {
        L.numel = {100, 7, 3000};
        for (int s = 0; s < kStreams; ++s) {
            L.ptr[s].clear();
            uint64_t a = ((uint64_t)1 << 40) + ((uint64_t)s << 36);
            for (int64_t n : L.numel) {
                L.ptr[s].push_back(fake(a));
                a += (uint64_t)(n * 4 + 64);
            }
        }
    };
    {
        List L; base(L); L.numel[1] = -1; expect_invalid(esz, L, "negative numel");
    }
    {
        List L; base(L); L.numel[1] = (int64_t)1 << 60; expect_invalid(esz, L, "huge numel");
    }
    {
        List L; base(L); L.shard_begin = 50; L.shard_end = 40; expect_invalid(esz, L, "reversed shard");
    }
    {
        List L; base(L); L.shard_end = 4000; expect_invalid(esz, L, "shard past the end");
    }
    {
        List L; base(L); L.shard_end = -2; expect_invalid(esz, L, "shard_end -2");
    }
    {
        List L; base(L); L.ptr[3][2] = nullptr; expect_invalid(esz, L, "null tensor pointer");
    }
    {
        List L; base(L); L.ptr[4][0] = fake(addr(L.ptr[4][0]) + 2); expect_invalid(esz, L, "misaligned fp32");
    }
    {
        List L; base(L); L.ptr[1].clear(); expect_invalid(esz, L, "null pointer array");
    }
    {
        List L; base(L); L.flat_mask = 1u << 12; expect_invalid(esz, L, "unknown flat_mask bit");
    }
    {
        List L; base(L); L.flat_mask = ADAMW_BLOCKED_STATE; L.ptr[2][0] = fake(addr(L.ptr[2][0]) + 8);
        expect_invalid(esz, L, "misaligned blocked buffer");
    }
    {
        List L; base(L); L.flat_mask = 1u << 2; L.shard_end = 50; L.ptr[2][0] = nullptr;
        expect_invalid(esz, L, "null flat buffer");
    }
    {
        List L; base(L);
        L.c = adamw_tensor_list{};
        const adamw_tensor_list* p = L.get();
        adamw_tensor_list copy = *p;
        copy.numel = nullptr;
        CHECK(build_plan(esz, &copy, 16384, kMaxUpdateChunks, &plan, err) == ADAMW_E_INVALID);
        copy = *p;
        copy.n_tensors = -3;
        CHECK(build_plan(esz, &copy, 16384, kMaxUpdateChunks, &plan, err) == ADAMW_E_INVALID);
    }
    {
        // bad chunk sizes and a chunk limit below the plan's size
        List L; base(L);
        CHECK(build_plan(esz, L.get(), 1000, kMaxUpdateChunks, &plan, err) == ADAMW_E_INVALID);
        CHECK(build_plan(esz, L.get(), 0, kMaxUpdateChunks, &plan, err) == ADAMW_E_INVALID);
        CHECK(build_plan(esz, L.get(), 16384, 2, &plan, err) == ADAMW_E_INVALID);
    }
    {
        // an empty list and an empty shard are valid and plan nothing
        List L;
        CHECK(build_plan(esz, L.get(), 16384, kMaxUpdateChunks, &plan, err) == ADAMW_OK && plan.chunks.empty());
        List M; base(M); M.shard_begin = M.shard_end = 60;
        CHECK(build_plan(esz, M.get(), 16384, kMaxUpdateChunks, &plan, err) == ADAMW_OK && plan.chunks.empty());
    }
}

void test_argument_checks()
{
    std::string err;
    adamw_hparams hp{2e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f};
    CHECK(check_hparams(&hp, err) == ADAMW_OK);
    CHECK(check_hparams(nullptr, err) == ADAMW_E_INVALID);
    const float bad[] = {-1.0f, 1.0f, 2.0f, __builtin_nanf(""), __builtin_inff(), -__builtin_inff()};
    for (int field = 0; field < 6; ++field) {
        for (float x : bad) {
            adamw_hparams h = hp;
            float* f = &h.lr + field;
            *f = x;
            const bool ok = check_hparams(&h, err) == ADAMW_OK;
            // lr, eps, wd may be any finite value >= 0; betas in [0, 1); inv scale > 0
            const bool want = x == x && x != __builtin_inff() && x != -__builtin_inff() && x >= 0.0f &&
                              !((field == 1 || field == 2) && x >= 1.0f) && !(field == 5 && x == 0.0f);
            CHECK(ok == want);
        }
    }
    adamw_loss_scaler sc{2.0f, 0.5f, 2000};
    CHECK(check_scaler(&sc, err) == ADAMW_OK);
    CHECK(check_scaler(nullptr, err) == ADAMW_E_INVALID);
    adamw_loss_scaler s2 = sc;
    s2.growth_factor = 0.5f;
    CHECK(check_scaler(&s2, err) == ADAMW_E_INVALID);
    s2 = sc;
    s2.backoff_factor = 0.0f;
    CHECK(check_scaler(&s2, err) == ADAMW_E_INVALID);
    s2 = sc;
    s2.growth_interval = 0;
    CHECK(check_scaler(&s2, err) == ADAMW_E_INVALID);
    CHECK(basic_list_check(nullptr, err) == ADAMW_E_INVALID);
    adamw_pure_precision pp{ADAMW_F32, ADAMW_BF16, 1};
    CHECK(check_pure_precision(&pp, err) == ADAMW_OK);
    CHECK(check_pure_precision(nullptr, err) == ADAMW_E_INVALID);
    pp.exp_avg = ADAMW_F16;
    CHECK(check_pure_precision(&pp, err) == ADAMW_E_UNSUPPORTED);
    // every mode / dtype pair the ABI can receive, valid or not
    for (int m = 0; m < 3; ++m)
        for (int d = 0; d < 3; ++d) {
            const adamw_status st = check_mode((adamw_mode)m, (adamw_dtype)d, false, err);
            const bool want = (m == ADAMW_MIXED && d != ADAMW_F32) || (m != ADAMW_MIXED && d == ADAMW_BF16);
            CHECK((st == ADAMW_OK) == want);
            int es[kStreams];
            mode_esizes((adamw_mode)m, (adamw_dtype)d, false, es);
            mix((uint64_t)(es[0] + 8 * es[2] + 64 * es[4]));
        }
}

// The plan cache of one stream, simulated with the library's slot policy:
// slots in most-recently-used order, each holding a list id; a pinned slot
// (captured by a graph) must keep its list whatever other lists come later.
void test_slot_policy()
{
    const size_t cap = 8;
    struct Slot { int list; bool pinned; };
    std::vector<Slot> slots;
    auto use = [&](int list, bool capture) {
        for (size_t i = 0; i < slots.size(); ++i)
            if (slots[i].list == list) {
                Slot s = slots[i];
                slots.erase(slots.begin() + (long)i);
                if (capture) s.pinned = true;
                slots.insert(slots.begin(), s);
                return;
            }
        CHECK(!capture);   // a capture never uploads a new table
        std::vector<bool> pinned;
        for (auto& s : slots) pinned.push_back(s.pinned);
        const size_t pick = choose_plan_slot(pinned, cap);
        CHECK(pick <= slots.size());
        if (pick == slots.size()) {
            slots.push_back(Slot{list, false});
        } else {
            CHECK(!slots[pick].pinned);
            slots[pick].list = list;
        }
        Slot s = slots[pick];
        slots.erase(slots.begin() + (long)pick);
        slots.insert(slots.begin(), s);
        size_t unpinned = 0;
        for (auto& x : slots) unpinned += !x.pinned;
        CHECK(unpinned <= cap);
    };
    // a captured list, then 11 other lists cycled through the cache 3 times
    use(100, false);
    use(100, true);
    for (int round = 0; round < 3; ++round)
        for (int l = 0; l < 11; ++l) use(l, false);
    bool found = false;
    for (auto& s : slots) found |= (s.list == 100 && s.pinned);
    CHECK(found);
    CHECK(slots.size() == cap + 1);
    // more captures: every pinned list stays; unpinned capacity stays at cap
    for (int l = 200; l < 205; ++l) {
        use(l, false);
        use(l, true);
    }
    for (int l = 0; l < 30; ++l) use(l, false);
    for (int l = 200; l < 205; ++l) {
        bool f = false;
        for (auto& s : slots) f |= (s.list == l && s.pinned);
        CHECK(f);
    }
    CHECK(slots.size() == cap + 6);
    // a policy choice over an all-pinned cache asks for a new slot
    CHECK(choose_plan_slot(std::vector<bool>(12, true), cap) == 12);
    CHECK(choose_plan_slot(std::vector<bool>(), cap) == 0);
    std::vector<bool> mixed = {false, true, false, true, false, false, false, false, false, false};
    CHECK(choose_plan_slot(mixed, cap) == 9);
    mixed[9] = true;
    CHECK(choose_plan_slot(mixed, cap) == 10);   // 7 unpinned < cap: a new slot
}

}  // namespace

int main()
{
    test_random_plans();
    test_copy_plans();
    test_invalid_lists();
    test_argument_checks();
    test_slot_policy();
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("plan_check ok %016llx\n", (unsigned long long)g_sum);
    return 0;
}
