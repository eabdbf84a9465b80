// pa_kvm.hip -- host-side KV page manager: free list, per-(slot, layer) block
// tables, admission credit and continuous / static batching.  Host code only
// (no kernels); it hands the decode and prefill kernels their block tables and
// lengths.
//
// What is managed (samir-vllm article, section "Gestion de la KV cache et
// strategies de batching"): one shared pool of physical 16-token pages; a block
// table per sequence and per layer; a request is admitted once its page budget
// is available, the budget being prompt_tokens + allowed_new_tokens - 1 tokens
// rounded up to whole 16-token pages, for each layer; a request whose budget
// exceeds the whole pool is refused with an explicit error instead of waiting
// forever.  Continuous batching admits requests as budgets free up; static
// batching waits until the running group has finished.  The initial state is
// the one tiny-vllm's chapter "Weight Loading and GPU Buffer Design" (section
// "What else is set up in the initialization block") describes: every page on
// the free list, every block-table entry -1, every batch slot free.
//
// Policies the pages leave open (stated here, tested in tests/test_kvm_host.py):
//  * Budgets are reserved at admission and pages are taken from the free list
//    only as a sequence grows, so growing within the budget never fails.
//  * The free list is a stack: page 0 is handed out first on a fresh pool and
//    the page returned last is reused first.
//  * Admission is first-come first-served: the queue head is admitted when its
//    budget and a slot are available; a head that does not fit yet blocks the
//    requests behind it (no overtaking, so a large request is never starved).
#include <stdint.h>
#include <stdlib.h>

#include <new>
#include <vector>

#include "pa.h"

struct pa_kv_manager {
    int32_t num_pages = 0;
    int32_t num_layers = 0;
    int32_t max_slots = 0;
    int32_t max_blocks = 0;
    int32_t batching = PA_BATCH_CONTINUOUS;
    std::vector<int32_t> free_stack;    // top = back
    std::vector<int32_t> block_tables;  // [layers][slots][max_blocks], -1 unassigned
    std::vector<int32_t> lengths;       // [slots] tokens with a page assigned (0 = free slot)
    std::vector<int32_t> budget_tokens; // [slots] prompt + max_new - 1 (0 = free slot)
    std::vector<int32_t> slot_request;  // [slots] request id or -1
    std::vector<int64_t> slot_credit;   // [slots] reserved pages (all layers)
    int64_t reserved = 0;               // pages reserved by admitted requests, not yet returned
    int64_t assigned = 0;               // pages currently in block tables
    struct Req {
        int32_t id, prompt, max_new;
        int64_t credit;
    };
    std::vector<Req> queue;  // FIFO, head = front
    size_t queue_head = 0;
    int32_t next_id = 0;
};

namespace {

int64_t credit_pages(int32_t prompt, int32_t max_new, int32_t layers) {
    if (prompt < 1 || max_new < 1 || layers < 1) return -1;
    const int64_t tokens = static_cast<int64_t>(prompt) + max_new - 1;
    return (tokens + PA_PAGE_SIZE - 1) / PA_PAGE_SIZE * layers;
}

int32_t active_slots(const pa_kv_manager *m) {
    int32_t n = 0;
    for (int32_t r : m->slot_request) n += r >= 0;
    return n;
}

int32_t free_slot(const pa_kv_manager *m) {
    for (int32_t s = 0; s < m->max_slots; ++s)
        if (m->slot_request[s] < 0) return s;
    return -1;
}

}  // namespace

extern "C" {

int64_t pa_admission_credit_pages(int32_t prompt_tokens, int32_t max_new_tokens, int32_t num_layers) {
    return credit_pages(prompt_tokens, max_new_tokens, num_layers);
}

pa_status pa_kvm_create(int32_t num_pages, int32_t num_layers, int32_t max_slots, int32_t max_blocks,
                        int32_t batching, pa_kv_manager **out) {
    if (!out) return PA_ERR_INVALID_ARG;
    *out = nullptr;
    if (num_pages < 1 || num_layers < 1 || max_slots < 1 || max_blocks < 1) return PA_ERR_INVALID_ARG;
    if (batching != PA_BATCH_CONTINUOUS && batching != PA_BATCH_STATIC) return PA_ERR_INVALID_ARG;
    const int64_t bt = static_cast<int64_t>(num_layers) * max_slots * max_blocks;
    if (bt > (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
    pa_kv_manager *m = new (std::nothrow) pa_kv_manager;
    if (!m) return PA_ERR_INVALID_ARG;
    try {
        m->num_pages = num_pages;
        m->num_layers = num_layers;
        m->max_slots = max_slots;
        m->max_blocks = max_blocks;
        m->batching = batching;
        m->free_stack.resize(num_pages);
        for (int32_t i = 0; i < num_pages; ++i) m->free_stack[i] = num_pages - 1 - i;  // page 0 on top
        m->block_tables.assign(static_cast<size_t>(bt), -1);
        m->lengths.assign(max_slots, 0);
        m->budget_tokens.assign(max_slots, 0);
        m->slot_request.assign(max_slots, -1);
        m->slot_credit.assign(max_slots, 0);
    } catch (...) {
        delete m;
        return PA_ERR_INVALID_ARG;
    }
    *out = m;
    return PA_OK;
}

void pa_kvm_destroy(pa_kv_manager *m) { delete m; }

pa_status pa_kvm_submit(pa_kv_manager *m, int32_t prompt_tokens, int32_t max_new_tokens, int32_t *request_id) {
    if (!m || !request_id) return PA_ERR_INVALID_ARG;
    *request_id = -1;
    const int64_t credit = credit_pages(prompt_tokens, max_new_tokens, m->num_layers);
    if (credit < 0) return PA_ERR_INVALID_ARG;
    const int64_t tokens = static_cast<int64_t>(prompt_tokens) + max_new_tokens - 1;
    // A budget the pool (or a block table) can never hold is refused now: waiting
    // for it would block the queue forever.
    if (credit > m->num_pages || tokens > static_cast<int64_t>(m->max_blocks) * PA_PAGE_SIZE)
        return PA_ERR_REJECTED;
    try {
        m->queue.push_back({m->next_id, prompt_tokens, max_new_tokens, credit});
    } catch (...) {
        return PA_ERR_INVALID_ARG;
    }
    *request_id = m->next_id++;
    return PA_OK;
}

int32_t pa_kvm_schedule(pa_kv_manager *m, int32_t *admitted_slots, int32_t max_out) {
    if (!m || max_out < 0 || (max_out > 0 && !admitted_slots)) return -1;
    if (m->batching == PA_BATCH_STATIC && active_slots(m) > 0) return 0;  // the group is still running
    int32_t n = 0;
    while (m->queue_head < m->queue.size() && n < max_out) {
        const pa_kv_manager::Req &r = m->queue[m->queue_head];
        const int32_t slot = free_slot(m);
        if (slot < 0 || r.credit > m->num_pages - m->reserved) break;
        m->slot_request[slot] = r.id;
        m->slot_credit[slot] = r.credit;
        m->budget_tokens[slot] = r.prompt + r.max_new - 1;
        m->lengths[slot] = 0;
        m->reserved += r.credit;
        admitted_slots[n++] = slot;
        ++m->queue_head;
    }
    if (m->queue_head == m->queue.size()) {  // drop the consumed prefix
        m->queue.clear();
        m->queue_head = 0;
    }
    return n;
}

pa_status pa_kvm_set_length(pa_kv_manager *m, int32_t slot, int32_t len) {
    if (!m || slot < 0 || slot >= m->max_slots || m->slot_request[slot] < 0) return PA_ERR_INVALID_ARG;
    if (len < m->lengths[slot] || len > m->budget_tokens[slot]) return PA_ERR_INVALID_ARG;
    const int32_t have = (m->lengths[slot] + PA_PAGE_SIZE - 1) / PA_PAGE_SIZE;
    const int32_t need = (len + PA_PAGE_SIZE - 1) / PA_PAGE_SIZE;
    // The reservation covers every page up to the budget, so the stack holds them.
    for (int32_t l = 0; l < m->num_layers; ++l) {
        int32_t *row = &m->block_tables[(static_cast<size_t>(l) * m->max_slots + slot) * m->max_blocks];
        for (int32_t b = have; b < need; ++b) {
            row[b] = m->free_stack.back();
            m->free_stack.pop_back();
            ++m->assigned;
        }
    }
    m->lengths[slot] = len;
    return PA_OK;
}

pa_status pa_kvm_release(pa_kv_manager *m, int32_t slot) {
    if (!m || slot < 0 || slot >= m->max_slots || m->slot_request[slot] < 0) return PA_ERR_INVALID_ARG;
    const int32_t have = (m->lengths[slot] + PA_PAGE_SIZE - 1) / PA_PAGE_SIZE;
    for (int32_t l = 0; l < m->num_layers; ++l) {
        int32_t *row = &m->block_tables[(static_cast<size_t>(l) * m->max_slots + slot) * m->max_blocks];
        for (int32_t b = have - 1; b >= 0; --b) {  // the sequence's first page ends on top
            m->free_stack.push_back(row[b]);
            row[b] = -1;
            --m->assigned;
        }
    }
    m->reserved -= m->slot_credit[slot];
    m->slot_credit[slot] = 0;
    m->slot_request[slot] = -1;
    m->lengths[slot] = 0;
    m->budget_tokens[slot] = 0;
    return PA_OK;
}

const int32_t *pa_kvm_block_tables(const pa_kv_manager *m) { return m ? m->block_tables.data() : nullptr; }
const int32_t *pa_kvm_lengths(const pa_kv_manager *m) { return m ? m->lengths.data() : nullptr; }
int32_t pa_kvm_slot_request(const pa_kv_manager *m, int32_t slot) {
    return (m && slot >= 0 && slot < m->max_slots) ? m->slot_request[slot] : -1;
}
int32_t pa_kvm_slot_budget(const pa_kv_manager *m, int32_t slot) {
    return (m && slot >= 0 && slot < m->max_slots) ? m->budget_tokens[slot] : -1;
}
int32_t pa_kvm_free_pages(const pa_kv_manager *m) { return m ? static_cast<int32_t>(m->free_stack.size()) : -1; }
int64_t pa_kvm_reserved_pages(const pa_kv_manager *m) { return m ? m->reserved : -1; }
int32_t pa_kvm_queued(const pa_kv_manager *m) {
    return m ? static_cast<int32_t>(m->queue.size() - m->queue_head) : -1;
}

}  // extern "C"
