"""Host KV page manager (pa_kvm_*): admission credit, refusal, batching
policies, free-list order and bookkeeping invariants.  No GPU needed.

What the pages fix (samir-vllm article, section "Gestion de la KV cache et
strategies de batching"): the admission credit is prompt_tokens +
allowed_new_tokens - 1 tokens rounded up to 16-token pages, for each layer; a
request whose budget exceeds the pool is refused with an explicit error;
continuous batching admits requests as their budgets become available, static
batching waits for the running group to finish.  tiny-vllm ch.2 ("What else is
set up ..."): all pages start free and every block-table entry at -1.  The
pages leave the page-choice and queue-order policies open; the ones the
library takes (stack free list, first-come first-served without overtaking)
are checked here as stated in include/pa.h.
"""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def pa():
    from paged_kv_gqa_append_amd import binding, build

    if not build.is_current():
        build.build()
    binding.lib()
    return binding


# Credit values worked out by hand from the rule on the page: tokens = prompt +
# new - 1, pages per layer = ceil(tokens / 16), times the layer count.
CREDIT_CASES = [
    # prompt, new, layers, pages
    (1, 1, 16, 16),        # 1 token -> 1 page per layer
    (16, 1, 16, 16),       # 16 tokens fill one page exactly
    (16, 2, 16, 32),       # 17 tokens spill into a second page
    (15, 2, 1, 1),         # 16 tokens, one layer
    (2000, 49, 16, 2048),  # 2048 tokens = 128 pages per layer
    (2000, 50, 16, 2064),  # 2049 tokens = 129 pages per layer
    (1, 1000, 3, 189),     # 1000 tokens = 63 pages per layer
]


@pytest.mark.parametrize("prompt,new,layers,pages", CREDIT_CASES)
def test_admission_credit_worked_examples(pa, prompt, new, layers, pages):
    assert pa.admission_credit_pages(prompt, new, layers) == pages


def test_admission_credit_invalid(pa):
    assert pa.admission_credit_pages(0, 5, 16) == -1
    assert pa.admission_credit_pages(5, 0, 16) == -1
    assert pa.admission_credit_pages(5, 5, 0) == -1


def test_initial_state(pa):
    m = pa.KVManager(num_pages=64, num_layers=2, max_slots=4, max_blocks=8)
    assert m.free_pages == 64 and m.reserved_pages == 0 and m.queued == 0
    assert (m.block_tables() == -1).all()
    assert (m.lengths() == 0).all()
    assert all(m.slot_request(s) == -1 for s in range(4))


def test_default_pool_refusal_boundary(pa):
    """samir-vllm's default pool is 128 MiB; at 2048 B per token per layer a
    16-token page of K and V is 32 KiB, so the pool holds 4096 pages.  Over 16
    layers that is 256 pages = 4096 tokens per sequence: a 4096-token budget is
    admitted, a 4097-token one is refused outright."""
    pool_pages = (128 << 20) // (16 * 2048)
    assert pool_pages == 4096
    m = pa.KVManager(num_pages=pool_pages, num_layers=16, max_slots=2, max_blocks=512)
    assert m.submit(4000, 97) >= 0            # 4096 tokens -> 256 x 16 = 4096 pages
    with pytest.raises(pa.PaError) as e:
        m.submit(4000, 98)                    # 4097 tokens -> 257 x 16 = 4112 pages
    assert e.value.status == pa.PA_ERR_REJECTED
    assert m.queued == 1


def test_refusal_beyond_block_table(pa):
    m = pa.KVManager(num_pages=10_000, num_layers=1, max_slots=2, max_blocks=128)
    assert m.submit(2000, 49) >= 0            # 2048 tokens = 128 blocks
    with pytest.raises(pa.PaError) as e:
        m.submit(2000, 50)                    # 2049 tokens need a 129th block
    assert e.value.status == pa.PA_ERR_REJECTED


def test_invalid_arguments(pa):
    with pytest.raises(pa.PaError):
        pa.KVManager(num_pages=0, num_layers=1, max_slots=1, max_blocks=1)
    with pytest.raises(pa.PaError):
        pa.KVManager(num_pages=8, num_layers=1, max_slots=1, max_blocks=1, batching=7)
    m = pa.KVManager(num_pages=8, num_layers=1, max_slots=1, max_blocks=4)
    with pytest.raises(pa.PaError):
        m.submit(0, 1)
    with pytest.raises(pa.PaError):
        m.set_length(0, 1)                    # slot not active
    with pytest.raises(pa.PaError):
        m.release(0)
    m.submit(10, 3)
    (slot,) = m.schedule()
    m.set_length(slot, 5)
    with pytest.raises(pa.PaError):
        m.set_length(slot, 4)                 # shrinking
    with pytest.raises(pa.PaError):
        m.set_length(slot, 13)                # budget is 10 + 3 - 1 = 12 tokens
    m.set_length(slot, 12)


def test_free_list_order_and_growth(pa):
    """Fresh pool: pages 0, 1, 2, ... in (layer, block) order as the slot grows;
    the budget is reserved at admission, pages are taken only as tokens arrive."""
    m = pa.KVManager(num_pages=32, num_layers=2, max_slots=2, max_blocks=4)
    m.submit(17, 10)                          # 26 tokens -> 2 pages per layer -> credit 4
    (slot,) = m.schedule()
    assert m.reserved_pages == 4 and m.free_pages == 32
    m.set_length(slot, 16)
    bt = m.block_tables()
    assert bt[0, slot].tolist() == [0, -1, -1, -1] and bt[1, slot].tolist() == [1, -1, -1, -1]
    m.set_length(slot, 17)                    # crosses into the second page
    bt = m.block_tables()
    assert bt[0, slot].tolist() == [0, 2, -1, -1] and bt[1, slot].tolist() == [1, 3, -1, -1]
    assert m.free_pages == 28 and m.lengths()[slot] == 17
    m.release(slot)
    assert m.free_pages == 32 and m.reserved_pages == 0 and (m.block_tables() == -1).all()
    # release pushes each layer's pages last-block-first (layer 0: 2, 0; layer 1:
    # 3, 1), so the stack top is 1, then 3: the page returned last is reused first
    m.submit(1, 1)
    (slot,) = m.schedule()
    m.set_length(slot, 1)
    assert m.block_tables()[0, slot, 0] == 1 and m.block_tables()[1, slot, 0] == 3


def test_continuous_batching_fifo(pa):
    m = pa.KVManager(num_pages=10, num_layers=1, max_slots=4, max_blocks=8, batching=pa.PA_BATCH_CONTINUOUS)
    a = m.submit(64, 1)      # 4 pages
    b = m.submit(80, 1)      # 5 pages
    c = m.submit(16, 1)      # 1 page
    d = m.submit(32, 1)      # 2 pages
    got = m.schedule()       # a (4) + b (5) + c (1) = 10 fit; d waits
    assert [m.slot_request(s) for s in got] == [a, b, c]
    assert m.reserved_pages == 10 and m.queued == 1
    assert m.schedule() == []
    m.release(got[2])        # c done: 1 page back, d needs 2 -> still waits
    assert m.schedule() == []
    m.release(got[0])        # a done: 5 unreserved -> d admitted into a free slot
    (s,) = m.schedule()
    assert m.slot_request(s) == d and m.reserved_pages == 7


def test_continuous_batching_no_overtaking(pa):
    m = pa.KVManager(num_pages=8, num_layers=1, max_slots=4, max_blocks=8)
    big0 = m.submit(96, 1)   # 6 pages
    big1 = m.submit(64, 1)   # 4 pages: does not fit next to big0
    small = m.submit(16, 1)  # 1 page: would fit, but must not overtake big1
    got = m.schedule()
    assert [m.slot_request(s) for s in got] == [big0]
    m.release(got[0])
    got = m.schedule()
    assert [m.slot_request(s) for s in got] == [big1, small]


def test_static_batching_waits_for_group(pa):
    m = pa.KVManager(num_pages=100, num_layers=1, max_slots=2, max_blocks=8, batching=pa.PA_BATCH_STATIC)
    ids = [m.submit(10, 5) for _ in range(5)]
    g1 = m.schedule()
    assert [m.slot_request(s) for s in g1] == ids[:2]           # slot-limited group
    m.release(g1[0])
    assert m.schedule() == []                                    # one member still running
    m.release(g1[1])
    g2 = m.schedule()
    assert [m.slot_request(s) for s in g2] == ids[2:4]


def test_slot_limit_continuous(pa):
    m = pa.KVManager(num_pages=100, num_layers=1, max_slots=2, max_blocks=8)
    ids = [m.submit(10, 5) for _ in range(3)]
    g = m.schedule()
    assert len(g) == 2
    m.release(g[1])
    (s,) = m.schedule()
    assert m.slot_request(s) == ids[2] and s == g[1]


def _check_invariants(m, active_len, credit_of):
    bt = m.block_tables()
    L, S, MB = bt.shape
    used = bt[bt >= 0]
    assert len(np.unique(used)) == len(used), "a page is assigned twice"
    assert used.min(initial=0) >= 0 and used.max(initial=0) < m.num_pages
    assert m.free_pages + len(used) == m.num_pages
    lens = m.lengths()
    for s in range(S):
        n = (lens[s] + 15) // 16
        assert (bt[:, s, :n] >= 0).all() and (bt[:, s, n:] == -1).all()
        if s not in active_len:
            assert lens[s] == 0 and m.slot_request(s) == -1
        else:
            assert lens[s] == active_len[s]
    assert m.reserved_pages == sum(credit_of[s] for s in active_len)
    assert m.reserved_pages <= m.num_pages


@pytest.mark.parametrize("batching", [0, 1])
def test_random_history_invariants(pa, batching):
    """A seeded history of submits, admissions, growth and releases: pages are
    never shared, the free count and reservations always add up, growth within
    the budget never fails, and admissions follow the FIFO rule exactly (a
    plain model of the queue, written from the rule, predicts every one)."""
    rng = np.random.default_rng(7 + batching)
    P, LAYERS, SLOTS, MB = 96, 3, 6, 16
    m = pa.KVManager(P, LAYERS, SLOTS, MB, batching=batching)
    queue, active_len, credit_of, budget_of, req_of = [], {}, {}, {}, {}
    for step in range(600):
        op = rng.integers(0, 4)
        if op == 0:
            prompt, new = int(rng.integers(1, 120)), int(rng.integers(1, 140))
            credit = -(-(prompt + new - 1) // 16) * LAYERS
            if credit > P or prompt + new - 1 > MB * 16:
                with pytest.raises(pa.PaError):
                    m.submit(prompt, new)
            else:
                rid = m.submit(prompt, new)
                queue.append((rid, credit, prompt + new - 1))
        elif op == 1:
            # model: admit heads in order while a slot is free and the credit fits
            expect = []
            if not (batching == 1 and active_len):
                free_slots = [s for s in range(SLOTS) if s not in active_len]
                reserved = sum(credit_of.values())
                while queue and free_slots and queue[0][1] <= P - reserved:
                    rid, credit, budget = queue.pop(0)
                    s = free_slots.pop(0)
                    expect.append((s, rid))
                    reserved += credit
                    active_len[s], credit_of[s], budget_of[s], req_of[s] = 0, credit, budget, rid
            got = m.schedule()
            assert [(s, m.slot_request(s)) for s in got] == expect
        elif op == 2 and active_len:
            s = int(rng.choice(sorted(active_len)))
            new_len = int(rng.integers(active_len[s], budget_of[s] + 1))
            m.set_length(s, new_len)
            active_len[s] = new_len
        elif op == 3 and active_len:
            s = int(rng.choice(sorted(active_len)))
            m.release(s)
            for d in (active_len, credit_of, budget_of, req_of):
                del d[s]
        _check_invariants(m, active_len, credit_of)
