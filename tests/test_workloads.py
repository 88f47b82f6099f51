"""The seeded input generator: determinism and the structure each workload promises."""
import math

import numpy as np
import pytest

import workloads as W


def test_same_seed_same_bits_any_thread_count():
    cfg = W.config(2).scaled(batch=8, lengths=("uniform", 100, 3000))
    a = W.make_workload(cfg, threads=1)
    b = W.make_workload(cfg, threads=4)
    for name in ("q", "k_pool", "v_pool", "page_table", "context_lens"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    c = W.make_workload(cfg, seed=99)
    assert not np.array_equal(a.k_pool, c.k_pool)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    from workloads.generate import _encode
    got = _encode(x.copy(), "bf16")
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... i.e. 0x3F82); above tie rounds up
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0x3F81]


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_config_structure(i):
    cfg = W.config(i)
    w = W.make_workload(cfg)
    B, Hq, D = w.q.shape
    NP, PS, Hkv, D2 = w.k_pool.shape
    assert (B, Hq, Hkv, D, PS) == (cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size)
    assert D2 == D and w.page_table.shape == (B, cfg.max_pages_per_seq)
    L = w.context_lens.astype(np.int64)
    n = -(-L // PS)
    used = [w.page_table[b, :n[b]] for b in range(B)]
    allp = np.concatenate(used)
    assert allp.min() >= 0 and allp.max() < NP
    if cfg.lengths[0] == "prefix":
        S = cfg.lengths[1] // PS
        assert all(np.array_equal(u[:S], used[0][:S]) for u in used)
        private = np.concatenate([u[S:] for u in used])
        assert len(set(private.tolist())) == len(private)
        assert not set(private.tolist()) & set(used[0][:S].tolist())
        total = S + len(private)
    else:
        assert len(set(allp.tolist())) == len(allp)   # drawn without replacement
        total = len(allp)
    if cfg.pool_pages is None:
        assert NP == math.ceil(1.1 * total)
    else:
        assert NP == cfg.pool_pages
    kind = cfg.lengths[0]
    drawn = w.append_lens if cfg.append else w.context_lens
    if kind == "uniform":
        assert drawn.min() >= cfg.lengths[1] and drawn.max() <= cfg.lengths[2]
    if kind == "loguniform":
        assert drawn.min() >= cfg.lengths[1] and drawn.max() <= cfg.lengths[2]
        assert np.median(drawn) < 0.5 * (cfg.lengths[1] + cfg.lengths[2])
    if cfg.append:
        assert np.array_equal(w.context_lens, w.append_lens + 1)
        assert w.k_new.shape == (B, Hkv, D)


def test_tiny_config_is_eight_pages_of_thirty_two():
    w = W.make_workload(W.config(1))
    assert w.k_pool.shape[0] == 32 and w.context_lens.tolist() == [128]
    assert len(set(w.page_table[0].tolist())) == 8


def test_config5_lengths_and_partitions():
    cfg = W.config(5)
    L = W.draw_lengths(cfg, cfg.index)
    assert L.min() >= 32768 and L.max() <= 131072 and cfg.partition_tokens == 4096


def test_poison_marks_unused_pages_and_tails():
    w = W.make_workload(W.config(1), poison=True)
    used = set(w.page_table[0].tolist())
    unused = [p for p in range(32) if p not in used]
    assert np.isnan(w.k_pool[unused]).all() and np.isnan(w.v_pool[unused]).all()
    assert not np.isnan(w.k_pool[list(used)]).any()   # L=128 fills every used page exactly
    w = W.make_workload(W.config(2).scaled(batch=3, lengths=("fixed", 20)), poison=True)
    last = w.page_table[:, 1]
    tail = w.k_pool[last, 4:]
    assert ((tail & 0x7FFF) > 0x7F80).all()     # bf16 NaN bits
    assert (w.page_table[:, 2:] == -1).all()


def test_relabel_and_unshare_keep_logical_rows():
    import oracle as O
    w = W.make_workload(W.config(3).scaled(batch=3, lengths=("prefix", 32, 1, 20)))
    for w2 in (W.relabel_pages(w, 5), W.unshare_prefix(w)):
        for b in range(3):
            L = int(w.context_lens[b])
            a = O.gather_rows(w.k_pool, w.page_table[b], L, 16)
            c = O.gather_rows(w2.k_pool, w2.page_table[b], L, 16)
            assert np.array_equal(a, c)
