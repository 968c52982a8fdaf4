// replay.hip -- sum-tree-backed replay priorities: a ring of `capacity`
// slots whose priorities live in an F32 sum tree.
//
// "GPU Segment Tree for PER Sampling", section "Integration with
// GpuReplayBuffer": inserting a batch writes its priorities and updates the
// tree at the inserted slots; updating priorities is the tree's batched
// update; proportional sampling is the root-to-leaf descent; the total
// priority is the root.  The ring (insert position advancing modulo the
// capacity, the number of filled slots) is host state in psamp_replay; every
// device step is an existing kernel (tree update, tree descent, IS weights)
// plus one small kernel that writes the inserted slot numbers.
#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

constexpr int64_t kTreeBatch = 1024;     // one tree update call takes at most this many

__global__ __launch_bounds__(256) void k_ring_slots(int32_t* __restrict__ out, int64_t m,
                                                   int64_t cursor, int64_t capacity) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < m) out[i] = (int32_t)((cursor + i) % capacity);
}

static psamp_status check_rb(const psamp_replay* rb) {
    if (!rb || !rb->tree) return PSAMP_E_NULL;
    if (rb->capacity < 1 || rb->cap_pow2 != psamp_segtree_cap_pow2(rb->capacity) ||
        rb->cursor < 0 || rb->cursor >= rb->capacity || rb->size < 0 ||
        rb->size > rb->capacity || !(rb->alpha > 0.0) || !finite_d(rb->alpha))
        return PSAMP_E_PARAM;
    return PSAMP_OK;
}

}  // namespace psamp

using namespace psamp;

// The workspace: the tree update's (its counter) first, then the IS
// weights' -- two regions, since both keep state from call to call.
static size_t upd_ws_bytes() { return psamp_segtree_update_workspace_size(1, 1); }

extern "C" size_t psamp_replay_workspace_size(int64_t capacity, int64_t max_batch) {
    const int64_t cp = psamp_segtree_cap_pow2(capacity);
    if (cp == 0 || max_batch < 0) return 0;
    return upd_ws_bytes() + psamp_is_weights_workspace_size(max_batch);
}

extern "C" psamp_status psamp_replay_init(psamp_replay* rb, int64_t capacity, double alpha,
                                          float* tree, void* ws, size_t ws_bytes) {
    if (!rb || !tree) return PSAMP_E_NULL;
    const int64_t cp = psamp_segtree_cap_pow2(capacity);
    if (cp == 0) return PSAMP_E_SIZE;
    if (!(alpha > 0.0) || !finite_d(alpha)) return PSAMP_E_PARAM;
    if (!aligned(tree, 16) || (ws && !aligned(ws, 8))) return PSAMP_E_ALIGN;
    rb->capacity = capacity;
    rb->cap_pow2 = cp;
    rb->cursor = 0;
    rb->size = 0;
    rb->alpha = alpha;
    rb->tree = tree;
    rb->ws = ws;
    rb->ws_bytes = ws ? ws_bytes : 0;
    return PSAMP_OK;
}

extern "C" psamp_status psamp_replay_insert(psamp_replay* rb, const float* prio, int64_t m,
                                            int32_t* out_slots, void* stream) {
    psamp_status s = check_rb(rb);
    if (s != PSAMP_OK) return s;
    if (!prio || !out_slots) return PSAMP_E_NULL;
    if (m < 0 || m > kMaxN) return PSAMP_E_SIZE;
    if (!aligned(prio, 4) || !aligned(out_slots, 4)) return PSAMP_E_ALIGN;
    if (m == 0) return PSAMP_OK;
    if (upd_ws_bytes() > rb->ws_bytes) return PSAMP_E_WORKSPACE;
    hipStream_t st = as_stream(stream);
    hipLaunchKernelGGL(k_ring_slots, dim3((unsigned)ceil_div(m, 256)), dim3(256), 0, st,
                       out_slots, m, rb->cursor, rb->capacity);
    s = launch_status();
    if (s != PSAMP_OK) return s;
    // in batch order, so a slot written twice keeps the later priority
    for (int64_t j = 0; j < m; j += kTreeBatch) {
        const int64_t c = m - j < kTreeBatch ? m - j : kTreeBatch;
        s = psamp_segtree_update(rb->tree, PSAMP_F32, rb->cap_pow2, out_slots + j, prio + j,
                                 PSAMP_F32, c, rb->alpha, rb->ws, rb->ws_bytes, stream);
        if (s != PSAMP_OK) return s;
    }
    rb->cursor = (rb->cursor + m) % rb->capacity;
    rb->size = rb->size + m < rb->capacity ? rb->size + m : rb->capacity;
    return PSAMP_OK;
}

extern "C" psamp_status psamp_replay_update(psamp_replay* rb, const int32_t* slots,
                                            const float* prio, int64_t m, void* stream) {
    psamp_status s = check_rb(rb);
    if (s != PSAMP_OK) return s;
    if (!slots || !prio) return PSAMP_E_NULL;
    if (m < 0 || m > kMaxN) return PSAMP_E_SIZE;
    if (m == 0) return PSAMP_OK;
    for (int64_t j = 0; j < m; j += kTreeBatch) {
        const int64_t c = m - j < kTreeBatch ? m - j : kTreeBatch;
        s = psamp_segtree_update(rb->tree, PSAMP_F32, rb->cap_pow2, slots + j, prio + j,
                                 PSAMP_F32, c, rb->alpha, rb->ws, rb->ws_bytes, stream);
        if (s != PSAMP_OK) return s;
    }
    return PSAMP_OK;
}

extern "C" psamp_status psamp_replay_sample(const psamp_replay* rb, const float* u, int64_t k,
                                            int stratified, double beta, int32_t* out_slots,
                                            float* out_w, void* stream) {
    psamp_status s = check_rb(rb);
    if (s != PSAMP_OK) return s;
    if (!u || !out_slots) return PSAMP_E_NULL;
    if (rb->size < 1 || k < 0 || k > kMaxN) return PSAMP_E_SIZE;
    if (stratified != 0 && stratified != 1) return PSAMP_E_PARAM;
    if (out_w && (!(beta >= 0.0) || !finite_d(beta))) return PSAMP_E_PARAM;
    if (k == 0) return PSAMP_OK;
    if (out_w && upd_ws_bytes() + psamp_is_weights_workspace_size(k) > rb->ws_bytes)
        return PSAMP_E_WORKSPACE;
    s = psamp_segtree_sample(rb->tree, PSAMP_F32, rb->cap_pow2, rb->size, u, PSAMP_F32, k,
                             stratified, out_slots, stream);
    if (s != PSAMP_OK || !out_w) return s;
    // the leaves already hold p^alpha: IS = (L_min / L_i)^beta
    return psamp_is_weights(rb->tree + rb->cap_pow2, PSAMP_F32, rb->size, 1.0, out_slots, k,
                            beta, out_w, (char*)rb->ws + upd_ws_bytes(),
                            rb->ws_bytes - upd_ws_bytes(), stream);
}

extern "C" const float* psamp_replay_total(const psamp_replay* rb) {
    return (rb && rb->tree) ? rb->tree + 1 : nullptr;
}
