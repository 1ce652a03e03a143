// Expert slot pools: the host side of streaming routed experts into a small
// per-layer pool of device slots (gfx950 host runtime, no kernels).
//
// Source: the anyesh.me page "Running a 26B MoE on an 8 GB Jetson by streaming
// experts from SSD", sections "Streaming without touching a single GPU kernel"
// and "Numbers from the actual machine".  Each MoE layer keeps a fixed number
// of expert-sized slots; when the router has chosen a token's experts, a
// per-layer LFU cache decides which are already resident (hits) and which
// slots the misses go to; the misses are read into their slots while the GPU
// runs the layer's shared dense work, and one join per layer makes the expert
// product wait for them.  The product itself is unchanged: it reads the pool
// through slot ids (w4_moe_gemv_ids with slot_of).
//
// Here the expert store is caller-owned pinned host memory and the reads are
// asynchronous host-to-device copies on a caller stream (the copy engines do
// the parallel reading that the page's small thread pool of file reads does).
//
// Ordering.  prepare(layer) enqueues on copy_stream, in order: a wait for the
// layer's last release (so no slot a previous product may still read is
// overwritten), the miss copies, the upload of the layer's slot map, and the
// layer's "copied" event.  join(layer) makes the compute stream wait for that
// event; release(layer) records, on the compute stream, the point after which
// the layer's pool and slot map may change again.
//
// LFU.  Per layer: a use count per expert (one per prepare call that requests
// it) and, per slot, its expert and the call that last used it.  A miss takes
// the lowest empty slot; when none is empty, the slot whose expert is not
// requested by this call and has the smallest use count, ties broken by the
// least recent use and then the lowest slot index.  Deterministic for a given
// sequence of requests.
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "w4.h"
#include "w4_internal.h"

struct w4_pool {
    int L = 0, E = 0, S = 0, P = 0;
    std::vector<int64_t> part_bytes;
    // per layer
    std::vector<std::vector<int32_t>> slot_of;   // [L][E], -1: not resident
    std::vector<std::vector<int32_t>> owner;     // [L][S], -1: empty
    std::vector<std::vector<uint64_t>> last_use; // [L][S]
    std::vector<std::vector<uint32_t>> uses;     // [L][E]
    std::vector<uint64_t> calls;                 // [L]: prepare/plan calls so far
    // device-side state, created on the first prepare
    bool dev_ready = false;
    std::vector<hipEvent_t> copied, released, uploaded;
    std::vector<char> released_set, uploaded_set;
    int32_t *pinned = nullptr;  // [2][L][E] staging of the slot maps (by call parity)
    int64_t hits = 0, misses = 0, bytes = 0;
};

namespace {

// The LFU decision for one call (host only).  miss_e / miss_s receive the
// misses in the order of the request; returns the miss count, or a negative
// status (nothing changed) when the request holds an invalid id or more
// distinct experts than slots.
int pool_plan(w4_pool *p, int layer, const int32_t *ids, int n_ids, std::vector<int32_t> &miss_e,
              std::vector<int32_t> &miss_s) {
    std::vector<char> want(p->E, 0);
    int distinct = 0;
    for (int i = 0; i < n_ids; ++i) {
        if (ids[i] < 0 || ids[i] >= p->E) return W4_ERR_INVALID_ARG;
        if (!want[ids[i]]) {
            want[ids[i]] = 1;
            ++distinct;
        }
    }
    if (distinct > p->S) return W4_ERR_UNSUPPORTED;
    auto &slot_of = p->slot_of[layer];
    auto &owner = p->owner[layer];
    auto &last = p->last_use[layer];
    auto &uses = p->uses[layer];
    const uint64_t now = ++p->calls[layer];
    miss_e.clear();
    miss_s.clear();
    for (int i = 0; i < n_ids; ++i) {
        const int e = ids[i];
        if (want[e] != 1) continue;  // each distinct expert once, in request order
        want[e] = 2;
        ++uses[e];
        if (slot_of[e] >= 0) {
            last[slot_of[e]] = now;
            ++p->hits;
            continue;
        }
        int victim = -1;
        for (int s = 0; s < p->S && victim < 0; ++s)
            if (owner[s] < 0) victim = s;
        if (victim < 0) {
            for (int s = 0; s < p->S; ++s) {
                const int o = owner[s];
                if (want[o]) continue;  // requested by this call: keep
                if (victim < 0 || uses[o] < uses[owner[victim]] ||
                    (uses[o] == uses[owner[victim]] && last[s] < last[victim]))
                    victim = s;
            }
        }
        // (distinct <= S guarantees a victim)
        if (owner[victim] >= 0) slot_of[owner[victim]] = -1;
        owner[victim] = e;
        slot_of[e] = victim;
        last[victim] = now;
        miss_e.push_back(e);
        miss_s.push_back(victim);
        ++p->misses;
    }
    return (int)miss_e.size();
}

int pool_device_init(w4_pool *p) {
    if (p->dev_ready) return W4_OK;
    p->copied.assign(p->L, nullptr);
    p->released.assign(p->L, nullptr);
    p->uploaded.assign(p->L * 2, nullptr);
    p->released_set.assign(p->L, 0);
    p->uploaded_set.assign(p->L * 2, 0);
    for (int l = 0; l < p->L; ++l) {
        if (hipEventCreateWithFlags(&p->copied[l], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&p->released[l], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&p->uploaded[2 * l], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&p->uploaded[2 * l + 1], hipEventDisableTiming) != hipSuccess)
            return W4_ERR_HIP;
    }
    void *h = nullptr;
    if (hipHostMalloc(&h, sizeof(int32_t) * 2 * (size_t)p->L * p->E, hipHostMallocDefault) != hipSuccess)
        return W4_ERR_HIP;
    p->pinned = static_cast<int32_t *>(h);
    p->dev_ready = true;
    return W4_OK;
}

}  // namespace

extern "C" {

int w4_pool_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, int32_t n_parts,
                   const int64_t *part_bytes, w4_pool **pool) {
    if (!pool) return W4_ERR_INVALID_ARG;
    *pool = nullptr;
    if (n_layers < 1 || n_experts < 1 || n_slots < 1 || n_parts < 1 || n_parts > W4_POOL_MAX_PARTS || !part_bytes)
        return W4_ERR_INVALID_ARG;
    for (int p = 0; p < n_parts; ++p)
        if (part_bytes[p] <= 0 || part_bytes[p] % 16) return W4_ERR_ALIGNMENT;
    w4_pool *p = new (std::nothrow) w4_pool;
    if (!p) return W4_ERR_UNSUPPORTED;
    p->L = n_layers;
    p->E = n_experts;
    p->S = n_slots;
    p->P = n_parts;
    p->part_bytes.assign(part_bytes, part_bytes + n_parts);
    p->slot_of.assign(n_layers, std::vector<int32_t>(n_experts, -1));
    p->owner.assign(n_layers, std::vector<int32_t>(n_slots, -1));
    p->last_use.assign(n_layers, std::vector<uint64_t>(n_slots, 0));
    p->uses.assign(n_layers, std::vector<uint32_t>(n_experts, 0));
    p->calls.assign(n_layers, 0);
    *pool = p;
    return W4_OK;
}

void w4_pool_destroy(w4_pool *p) {
    if (!p) return;
    if (p->dev_ready) {
        // the pinned staging may still be read by queued copies
        for (hipEvent_t e : p->uploaded) (void)hipEventSynchronize(e);
        for (hipEvent_t e : p->copied) (void)hipEventDestroy(e);
        for (hipEvent_t e : p->released) (void)hipEventDestroy(e);
        for (hipEvent_t e : p->uploaded) (void)hipEventDestroy(e);
        (void)hipHostFree(p->pinned);
    }
    delete p;
}

int w4_pool_plan(w4_pool *p, int32_t layer, const int32_t *ids, int32_t n_ids, int32_t *slot_of_out,
                 int32_t *miss_expert, int32_t *miss_slot) {
    if (!p || layer < 0 || layer >= p->L || n_ids < 0 || (n_ids > 0 && !ids)) return W4_ERR_INVALID_ARG;
    std::vector<int32_t> me, ms;
    const int nm = pool_plan(p, layer, ids, n_ids, me, ms);
    if (nm < 0) return nm;
    if (slot_of_out) std::memcpy(slot_of_out, p->slot_of[layer].data(), sizeof(int32_t) * p->E);
    for (int i = 0; i < nm; ++i) {
        if (miss_expert) miss_expert[i] = me[i];
        if (miss_slot) miss_slot[i] = ms[i];
    }
    return nm;
}

int w4_pool_prepare(w4_pool *p, int32_t layer, const int32_t *ids, int32_t n_ids, const void *const *host_parts,
                    void *const *dev_parts, int32_t *dev_slot_of, void *copy_stream) {
    if (!p || layer < 0 || layer >= p->L || n_ids < 0 || (n_ids > 0 && !ids) || !host_parts || !dev_parts ||
        !dev_slot_of)
        return W4_ERR_INVALID_ARG;
    for (int q = 0; q < p->P; ++q)
        if (!host_parts[q] || !dev_parts[q]) return W4_ERR_INVALID_ARG;
    int st = pool_device_init(p);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(copy_stream);
    // the slot-map staging of this parity was last read two calls ago
    const int par = (int)(p->calls[layer] & 1);
    hipEvent_t &up = p->uploaded[2 * layer + par];
    if (p->uploaded_set[2 * layer + par] && hipEventSynchronize(up) != hipSuccess) return W4_ERR_HIP;
    std::vector<int32_t> me, ms;
    const int nm = pool_plan(p, layer, ids, n_ids, me, ms);
    if (nm < 0) return nm;
    if (w4::settings().force_launch_error) return W4_ERR_HIP;
    if (p->released_set[layer] && hipStreamWaitEvent(s, p->released[layer], 0) != hipSuccess) return W4_ERR_HIP;
    for (int i = 0; i < nm; ++i) {
        for (int q = 0; q < p->P; ++q) {
            const int64_t b = p->part_bytes[q];
            const char *src = static_cast<const char *>(host_parts[q]) + (int64_t)me[i] * b;
            char *dst = static_cast<char *>(dev_parts[q]) + (int64_t)ms[i] * b;
            if (hipMemcpyAsync(dst, src, (size_t)b, hipMemcpyHostToDevice, s) != hipSuccess) return W4_ERR_HIP;
            p->bytes += b;
        }
    }
    int32_t *stage = p->pinned + ((size_t)par * p->L + layer) * p->E;
    std::memcpy(stage, p->slot_of[layer].data(), sizeof(int32_t) * p->E);
    if (hipMemcpyAsync(dev_slot_of, stage, sizeof(int32_t) * p->E, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipEventRecord(up, s) != hipSuccess || hipEventRecord(p->copied[layer], s) != hipSuccess)
        return W4_ERR_HIP;
    p->uploaded_set[2 * layer + par] = 1;
    return W4_OK;
}

int w4_pool_join(w4_pool *p, int32_t layer, void *stream) {
    if (!p || layer < 0 || layer >= p->L || !p->dev_ready) return W4_ERR_INVALID_ARG;
    return hipStreamWaitEvent(static_cast<hipStream_t>(stream), p->copied[layer], 0) == hipSuccess ? W4_OK
                                                                                                    : W4_ERR_HIP;
}

int w4_pool_release(w4_pool *p, int32_t layer, void *stream) {
    if (!p || layer < 0 || layer >= p->L || !p->dev_ready) return W4_ERR_INVALID_ARG;
    if (hipEventRecord(p->released[layer], static_cast<hipStream_t>(stream)) != hipSuccess) return W4_ERR_HIP;
    p->released_set[layer] = 1;
    return W4_OK;
}

int w4_pool_stats(const w4_pool *p, int64_t *hits, int64_t *misses, int64_t *bytes) {
    if (!p) return W4_ERR_INVALID_ARG;
    if (hits) *hits = p->hits;
    if (misses) *misses = p->misses;
    if (bytes) *bytes = p->bytes;
    return W4_OK;
}

}  // extern "C"
