"""Pins of the fp64 oracle against things other than itself.

No page prints a numeric example of paged attention, so every pin here is by construction:
loop-only brute force over contiguous K/V built without any pool, closed forms, invariants and
special cases.  Each is chosen so that a plausible slip in the oracle (a dropped max subtraction,
a wrong page/slot index, a transposed operand, a wrong GQA head map, a dropped partition) fails.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------------
# helpers: build a paged pool from logical rows (test-side scatter), and a loop-only brute force
# ----------------------------------------------------------------------------------------------

def scatter_to_pool(rows_per_seq, page_size, pool_pages, rng, fill=np.nan, dtype=np.float64):
    """rows_per_seq[b]: [L_b, Hkv, D].  Pages are taken from a random permutation of the pool."""
    Hkv, D = rows_per_seq[0].shape[1:]
    pool = np.full((pool_pages, page_size, Hkv, D), fill, dtype=dtype)
    perm = list(rng.permutation(pool_pages))
    n_max = max(-(-len(r) // page_size) for r in rows_per_seq)
    table = np.full((len(rows_per_seq), max(n_max, 1)), -1, dtype=np.int32)
    for b, rows in enumerate(rows_per_seq):
        for i in range(-(-len(rows) // page_size)):
            page = perm.pop()
            table[b, i] = page
            chunk = rows[i * page_size:(i + 1) * page_size]
            pool[page, :len(chunk)] = chunk
    return pool, table


def brute_decode(q, K_log, V_log, scale):
    """Loop-only attention: q [Hq][D]; K_log, V_log [L][Hkv][D] (nested lists)."""
    Hq = len(q)
    Hkv = len(K_log[0])
    G = Hq // Hkv
    out = []
    lses = []
    for h in range(Hq):
        kv = h // G
        s = [scale * math.fsum(q[h][d] * K_log[t][kv][d] for d in range(len(q[h])))
             for t in range(len(K_log))]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        out.append([math.fsum(w[t] * V_log[t][kv][d] for t in range(len(w))) / z
                    for d in range(len(V_log[0][0]))])
        lses.append(m + math.log(z))
    return out, lses


def run_oracle_f64(q, pool_k, pool_v, table, lens, scale):
    return O.paged_decode_attention(q.astype(np.float32), pool_k.astype(np.float32),
                                    pool_v.astype(np.float32), table, lens, scale, "f32")


# ----------------------------------------------------------------------------------------------
# element decoding
# ----------------------------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x4B80],
                    dtype=np.uint16)
    got = O.to_f64(bits, "bf16")
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, math.inf, -math.inf, 0.0, -0.0, 16777216.0]
    assert list(got) == want
    assert math.copysign(1.0, got[7]) == -1.0
    assert np.isnan(O.to_f64(np.array([0x7FC0], dtype=np.uint16), "bf16"))[0]


def test_bf16_decode_matches_bytewise_float32():
    """Independent path: build the float32 from its big-endian bytes with ``struct``."""
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=2000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    got = O.to_f64(bits, "bf16")
    for b, g in zip(bits, got):
        ref = struct.unpack(">f", bytes([int(b) >> 8, int(b) & 0xFF, 0, 0]))[0]
        assert g == ref


def test_f16_decode_exact():
    vals = np.array([1.0, -2.5, 65504.0, 2.0 ** -24, 0.1], dtype=np.float16)
    got = O.to_f64(vals, "f16")
    assert got[0] == 1.0 and got[1] == -2.5 and got[2] == 65504.0 and got[3] == 2.0 ** -24
    assert got[4] == float(np.float16(0.1))


# ----------------------------------------------------------------------------------------------
# brute force on tiny inputs
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_oracle_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 4))
    D = int(rng.choice([3, 5, 8]))
    PS = int(rng.choice([2, 3, 4]))
    Hq = Hkv * G
    lens = rng.integers(1, 40, size=B)
    K_log = [rng.standard_normal((L, Hkv, D)).astype(np.float32).astype(np.float64) for L in lens]
    V_log = [rng.standard_normal((L, Hkv, D)).astype(np.float32).astype(np.float64) for L in lens]
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    scale = np.float32(0.37)
    pool_pages = sum(-(-int(L) // PS) for L in lens) + 3
    pk, table = scatter_to_pool(K_log, PS, pool_pages, np.random.default_rng(seed))
    pv, table2 = scatter_to_pool(V_log, PS, pool_pages, np.random.default_rng(seed))
    assert np.array_equal(table, table2)
    out, lse = run_oracle_f64(q, pk, pv, table, lens.astype(np.int32), scale)
    for b in range(B):
        bo, bl = brute_decode(q[b].astype(np.float64).tolist(), K_log[b].tolist(),
                              V_log[b].tolist(), float(scale))
        np.testing.assert_allclose(out[b], np.array(bo), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], np.array(bl), rtol=0, atol=1e-12)


def test_oracle_bf16_matches_brute_force():
    """bf16 storage: the brute force decodes bits through ``struct`` rather than the oracle."""
    rng = np.random.default_rng(7)
    B, Hkv, G, D, PS = 2, 2, 2, 8, 4
    lens = np.array([13, 6], dtype=np.int32)
    pool_pages = 8
    w = W.make_workload(W.config(2).scaled(batch=2, lengths=("fixed", 13)), seed=3)
    # synthetic bf16 bits in a pool built by hand
    kb = rng.integers(0x3000, 0x4000, size=(pool_pages, PS, Hkv, D)).astype(np.uint16)
    vb = rng.integers(0xB000, 0xC000, size=(pool_pages, PS, Hkv, D)).astype(np.uint16)
    qb = rng.integers(0x3C00, 0x4000, size=(B, Hkv * G, D)).astype(np.uint16)
    table = np.array([[5, 1, 7, 2], [3, 0, 0, 0]], dtype=np.int32)
    dec = np.vectorize(lambda u: struct.unpack(">f", bytes([int(u) >> 8, int(u) & 0xFF, 0, 0]))[0])
    out, lse = O.paged_decode_attention(qb, kb, vb, table, lens, np.float32(0.25), "bf16")
    for b in range(B):
        L = int(lens[b])
        K_log = [[dec(kb[table[b, t // PS], t % PS, h]).tolist() for h in range(Hkv)] for t in range(L)]
        V_log = [[dec(vb[table[b, t // PS], t % PS, h]).tolist() for h in range(Hkv)] for t in range(L)]
        bo, bl = brute_decode(dec(qb[b]).tolist(), K_log, V_log, 0.25)
        np.testing.assert_allclose(out[b], np.array(bo), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], np.array(bl), rtol=0, atol=1e-12)
    assert w.q.dtype == np.uint16


# ----------------------------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------------------------

def _tiny_pool(K_rows, V_rows, PS=4, perm_seed=0, pool_extra=2):
    K_log = [np.asarray(K_rows, dtype=np.float64)]
    V_log = [np.asarray(V_rows, dtype=np.float64)]
    n = -(-len(K_rows) // PS) + pool_extra
    pk, t = scatter_to_pool(K_log, PS, n, np.random.default_rng(perm_seed))
    pv, _ = scatter_to_pool(V_log, PS, n, np.random.default_rng(perm_seed))
    return pk, pv, t


def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((1, 1, 6)).astype(np.float32)
    V = rng.standard_normal((1, 1, 6)).astype(np.float32)
    pk, pv, t = _tiny_pool(K, V)
    q = rng.standard_normal((1, 1, 6)).astype(np.float32)
    out, lse = run_oracle_f64(q, pk, pv, t, np.array([1], np.int32), np.float32(0.5))
    assert np.array_equal(out[0, 0], V[0, 0].astype(np.float64))
    assert lse[0, 0] == pytest.approx(0.5 * float(np.dot(q[0, 0].astype(np.float64), K[0, 0])), abs=1e-12)


def test_two_tokens_sigmoid_closed_form():
    # scale 1, q = e0, so the scores are exactly the first K component: 0.75 and -0.25
    K = np.array([[[0.75, 9.0, -3.0]], [[-0.25, 4.0, 1.0]]], dtype=np.float32)
    V = np.array([[[1.0, -2.0, 0.5]], [[3.0, 0.25, -1.0]]], dtype=np.float32)
    pk, pv, t = _tiny_pool(K, V, PS=1)
    q = np.array([[[1.0, 0.0, 0.0]]], dtype=np.float32)
    out, lse = run_oracle_f64(q, pk, pv, t, np.array([2], np.int32), np.float32(1.0))
    a = 1.0 / (1.0 + math.exp(-1.0))   # sigma(s1 - s2), s1 - s2 = 1
    want = a * V[0, 0].astype(np.float64) + (1 - a) * V[1, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(0.75) + math.exp(-0.25)), abs=1e-15)


def test_constant_values_return_the_constant():
    rng = np.random.default_rng(2)
    L = 37
    K = rng.standard_normal((L, 1, 8)).astype(np.float32)
    V = np.full((L, 1, 8), -1.375, dtype=np.float32)
    pk, pv, t = _tiny_pool(K, V, PS=4)
    q = rng.standard_normal((1, 1, 8)).astype(np.float32) * 3
    out, _ = run_oracle_f64(q, pk, pv, t, np.array([L], np.int32), np.float32(0.7))
    np.testing.assert_allclose(out[0, 0], -1.375, rtol=0, atol=1e-15)


@pytest.mark.parametrize("which", ["zero_q", "zero_scale", "identical_keys", "huge_equal_scores"])
def test_uniform_weights_give_mean_of_values(which):
    rng = np.random.default_rng(3)
    L, D = 29, 5
    K = rng.standard_normal((L, 1, D)).astype(np.float32)
    V = rng.standard_normal((L, 1, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    scale = np.float32(0.5)
    if which == "zero_q":
        q[:] = 0
    elif which == "zero_scale":
        scale = np.float32(0.0)
    elif which == "identical_keys":
        K[:] = K[0]
    else:  # every score equals 1600: exp overflows unless the max is subtracted first
        K[:] = 0
        K[:, :, 0] = 40.0
        q[:] = 0
        q[0, 0, 0] = 80.0
    pk, pv, t = _tiny_pool(K, V, PS=3)
    out, lse = run_oracle_f64(q, pk, pv, t, np.array([L], np.int32), scale)
    mean = [math.fsum(V[i, 0, d] for i in range(L)) / L for d in range(D)]
    np.testing.assert_allclose(out[0, 0], mean, rtol=0, atol=1e-13)
    s0 = float(scale) * float(np.dot(q[0, 0].astype(np.float64), K[0, 0].astype(np.float64)))
    assert lse[0, 0] == pytest.approx(s0 + math.log(L), abs=1e-10)


@pytest.mark.parametrize("PS", [2, 4, 16])
def test_address_probe_every_slot(PS):
    """One token scores 0, every other scores <= -1e4: the output is exactly that token's V row."""
    rng = np.random.default_rng(4)
    L, D = 3 * PS + 1, 4
    V = rng.standard_normal((L, 1, D)).astype(np.float32)
    pool_pages = 6
    for t_star in range(L):
        K = np.zeros((L, 1, D), dtype=np.float32)
        K[:, 0, 0] = -1e4
        K[t_star, 0, 0] = 0.0
        pk, pv, t = _tiny_pool(K, V, PS=PS, perm_seed=t_star, pool_extra=pool_pages - (-(-L // PS)))
        q = np.array([[[1.0, 0, 0, 0]]], dtype=np.float32)
        out, _ = run_oracle_f64(q, pk, pv, t, np.array([L], np.int32), np.float32(1.0))
        assert np.array_equal(out[0, 0], V[t_star, 0].astype(np.float64)), t_star


def test_empty_rows_give_zero_and_minus_inf():
    w = W.make_workload(W.config(2).scaled(batch=4, lengths=("uniform", 20, 70)), pad_rows=[1, 3])
    out, lse = O.paged_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table, w.context_lens,
                                        w.scale, w.dtype)
    assert np.all(out[[1, 3]] == 0) and np.all(lse[[1, 3]] == -np.inf)
    assert np.all(np.isfinite(out[[0, 2]]))


# ----------------------------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------------------------

def test_gqa_equals_mha_over_repeated_kv_heads():
    """Query head h reads KV head h // G: expanding each KV head G times gives the same result
    through the G = 1 (multi-head) path."""
    w = W.make_workload(W.config(4).scaled(batch=3, lengths=("uniform", 40, 90)))
    G = w.cfg.group
    out, lse = O.paged_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table, w.context_lens,
                                        w.scale, w.dtype)
    kx = np.repeat(w.k_pool, G, axis=2)
    vx = np.repeat(w.v_pool, G, axis=2)
    out2, lse2 = O.paged_decode_attention(w.q, kx, vx, w.page_table, w.context_lens, w.scale, w.dtype)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-14)
    # and heads of one group given the same query agree
    q = w.q.copy()
    q[:, 1] = q[:, 0]
    o3, _ = O.paged_decode_attention(q, w.k_pool, w.v_pool, w.page_table, w.context_lens, w.scale, w.dtype)
    assert np.array_equal(o3[:, 0], o3[:, 1])
    assert not np.allclose(o3[:, 0], o3[:, G])   # a different KV head gives a different answer


def test_page_relabelling_invariance():
    w = W.make_workload(W.config(2).scaled(batch=5, lengths=("uniform", 1, 100)))
    w2 = W.relabel_pages(w, seed=9)
    assert not np.array_equal(w.page_table, w2.page_table)
    a = O.paged_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table, w.context_lens, w.scale, w.dtype)
    b = O.paged_decode_attention(w2.q, w2.k_pool, w2.v_pool, w2.page_table, w2.context_lens, w2.scale, w2.dtype)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_shared_prefix_matches_unshared_copies():
    w = W.make_workload(W.config(3).scaled(batch=4, lengths=("prefix", 64, 5, 40)))
    assert w.shared_pages == 4
    assert len({tuple(w.page_table[b, :4]) for b in range(4)}) == 1
    u = W.unshare_prefix(w)
    assert len({tuple(u.page_table[b, :4]) for b in range(4)}) == 4
    a = O.paged_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table, w.context_lens, w.scale, w.dtype)
    b = O.paged_decode_attention(u.q, u.k_pool, u.v_pool, u.page_table, u.context_lens, u.scale, u.dtype)
    assert np.array_equal(a[0], b[0])


def test_poison_never_reaches_the_result():
    cfg = W.config(2).scaled(batch=6, lengths=("uniform", 3, 75))
    clean = W.make_workload(cfg)
    bad = W.make_workload(cfg, poison=True)
    assert np.isnan(O.to_f64(bad.k_pool, "bf16")).any() and (bad.page_table < 0).any()
    a = O.paged_decode_attention(clean.q, clean.k_pool, clean.v_pool, clean.page_table,
                                 clean.context_lens, clean.scale, clean.dtype)
    b = O.paged_decode_attention(bad.q, bad.k_pool, bad.v_pool, bad.page_table,
                                 bad.context_lens, bad.scale, bad.dtype)
    assert np.array_equal(a[0], b[0])


# ----------------------------------------------------------------------------------------------
# split-KV partitions and the log-sum-exp merge
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("P", [16, 32, 48])
def test_lse_merge_of_partials_is_the_full_result(P):
    w = W.make_workload(W.config(5).scaled(batch=3, lengths=("uniform", 1, 150)))
    full_o, full_l = O.paged_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table,
                                              w.context_lens, w.scale, w.dtype)
    po, pl = O.paged_decode_attention_partial(w.q, w.k_pool, w.v_pool, w.page_table,
                                              w.context_lens, w.scale, w.dtype, P)
    n = O.num_partitions(w.context_lens, P)
    assert po.shape[2] == n.max() and n.max() > 1
    mo, ml = O.lse_merge(po, pl, n)
    np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)


def test_each_partition_is_attention_over_its_own_tokens():
    w = W.make_workload(W.config(5).scaled(batch=2, lengths=("fixed", 40)))
    P = 16
    po, pl = O.paged_decode_attention_partial(w.q, w.k_pool, w.v_pool, w.page_table,
                                              w.context_lens, w.scale, w.dtype, P)
    for p, (lo, hi) in enumerate([(0, 16), (16, 32), (32, 40)]):
        # brute force over exactly tokens [lo, hi), built from the pool by explicit (page, slot)
        for b in range(2):
            Kl, Vl = [], []
            for t in range(lo, hi):
                page, slot = w.page_table[b, t // 16], t % 16
                Kl.append(O.to_f64(w.k_pool[page, slot], "bf16").tolist())
                Vl.append(O.to_f64(w.v_pool[page, slot], "bf16").tolist())
            bo, bl = brute_decode(O.to_f64(w.q[b], "bf16").tolist(), Kl, Vl, float(w.scale))
            np.testing.assert_allclose(po[b, :, p], np.array(bo), rtol=0, atol=1e-12)
            np.testing.assert_allclose(pl[b, :, p], np.array(bl), rtol=0, atol=1e-12)


def test_single_partition_merge_is_identity():
    rng = np.random.default_rng(5)
    po = rng.standard_normal((2, 3, 4, 8))
    pl = rng.standard_normal((2, 3, 4))
    mo, ml = O.lse_merge(po, pl, np.array([1, 1]))
    assert np.array_equal(mo, po[:, :, 0]) and np.array_equal(ml, pl[:, :, 0])
    mo, ml = O.lse_merge(po, pl, np.array([0, 2]))
    assert np.all(mo[0] == 0) and np.all(ml[0] == -np.inf)


# ----------------------------------------------------------------------------------------------
# append
# ----------------------------------------------------------------------------------------------

def _append_checks(w, kp, vp):
    """The appended row sits at logical position L of row b; every other byte is unchanged."""
    PS = w.k_pool.shape[1]
    touched = np.zeros(w.k_pool.shape[:2], dtype=bool)
    for b in range(w.q.shape[0]):
        L = int(w.append_lens[b])
        if L < 0:
            continue
        rows = O.gather_rows(kp, w.page_table[b], L + 1, PS)
        if not np.array_equal(rows[L].view(np.uint8), w.k_new[b].view(np.uint8)):
            return False
        rows = O.gather_rows(vp, w.page_table[b], L + 1, PS)
        if not np.array_equal(rows[L].view(np.uint8), w.v_new[b].view(np.uint8)):
            return False
        touched[w.page_table[b, L // PS], L % PS] = True
    same = ~touched
    return (np.array_equal(kp[same].view(np.uint8), w.k_pool[same].view(np.uint8))
            and np.array_equal(vp[same].view(np.uint8), w.v_pool[same].view(np.uint8)))


def test_append_writes_exactly_one_row_per_sequence():
    w = W.make_workload(W.config(4).scaled(batch=6, lengths=("loguniform", 1, 200)), pad_rows=[2])
    kp, vp = O.paged_kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.page_table, w.append_lens)
    assert _append_checks(w, kp, vp)
    assert not np.array_equal(kp, w.k_pool)
    kp2, vp2 = O.paged_kv_append(kp, vp, w.k_new, w.v_new, w.page_table, w.append_lens)
    assert np.array_equal(kp2.view(np.uint8), kp.view(np.uint8))   # idempotent


def test_append_negative_control_off_by_one_is_caught(monkeypatch):
    """A planted off-by-one slot in the oracle's append must fail the byte checks above."""
    w = W.make_workload(W.config(4).scaled(batch=4, lengths=("uniform", 5, 60)))

    def shifted(k_pool, v_pool, k_new, v_new, page_table, append_lens):
        kp, vp = k_pool.copy(), v_pool.copy()
        PS = k_pool.shape[1]
        for b, L in enumerate(append_lens):
            L = int(L) + 1   # planted mistake
            kp[page_table[b, L // PS], L % PS] = k_new[b]
            vp[page_table[b, L // PS], L % PS] = v_new[b]
        return kp, vp

    monkeypatch.setattr(O, "paged_kv_append", shifted)
    kp, vp = O.paged_kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.page_table, w.append_lens)
    assert not _append_checks(w, kp, vp)


def test_append_then_attend_sees_the_new_row():
    w = W.make_workload(W.config(4).scaled(batch=3, lengths=("fixed", 31)))
    kp, vp = O.paged_kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.page_table, w.append_lens)
    out, _ = O.paged_decode_attention(w.q, kp, vp, w.page_table, w.context_lens, w.scale, w.dtype)
    out_old, _ = O.paged_decode_attention(w.q, w.k_pool, w.v_pool, w.page_table, w.context_lens,
                                          w.scale, w.dtype)
    assert not np.allclose(out, out_old)
    assert np.all(w.context_lens == w.append_lens + 1)


# ----------------------------------------------------------------------------------------------
# metadata validation
# ----------------------------------------------------------------------------------------------

def test_validate_metadata_flags():
    w = W.make_workload(W.config(4).scaled(batch=4, lengths=("uniform", 5, 60)))
    NP, PS = w.k_pool.shape[:2]
    assert O.validate_metadata(w.page_table, w.append_lens, NP, PS, 1, True) == 0
    t = w.page_table.copy()
    t[1, 0] = NP
    assert O.validate_metadata(t, w.append_lens, NP, PS, 1) == O.STATUS_PAGE_RANGE
    lens = w.append_lens.copy()
    lens[0] = t.shape[1] * PS
    assert O.validate_metadata(w.page_table, lens, NP, PS, 1) & O.STATUS_CAPACITY
    t = w.page_table.copy()
    L0 = int(w.append_lens[0])
    t[0, L0 // PS] = t[1, 0]
    assert O.validate_metadata(t, w.append_lens, NP, PS, 1, True) & O.STATUS_APPEND_ALIAS


# ----------------------------------------------------------------------------------------------
# hand-derived golden example
# ----------------------------------------------------------------------------------------------

def test_golden_hand_derived_example():
    with open(os.path.join(GOLDEN, "paged_two_head_exact.json")) as f:
        g = json.load(f)
    k_pool = np.array(g["k_pool"], dtype=np.float32)
    v_pool = np.array(g["v_pool"], dtype=np.float32)
    q = np.array(g["q"], dtype=np.float32)
    table = np.array(g["page_table"], dtype=np.int32)
    lens = np.array(g["context_lens"], dtype=np.int32)
    out, lse = O.paged_decode_attention(q, k_pool, v_pool, table, lens, np.float32(g["scale"]), "f32")
    np.testing.assert_allclose(out, np.array(g["expected_out"]), rtol=0, atol=1e-15)
    want_lse = [[a + math.log(n) for a, n in row] for row in g["expected_lse"]]
    np.testing.assert_allclose(lse, np.array(want_lse), rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------------------------
# multi-query (causal) decode
# ----------------------------------------------------------------------------------------------

def brute_causal(qs, K_log, V_log, scale):
    """Loop-only causal attention of T queries qs [T][Hq][D] that are the last T tokens of the
    sequence K_log/V_log [L][Hkv][D]: query j sees rows 0 .. L - T + j (an explicit mask)."""
    T, L = len(qs), len(K_log)
    outs = []
    for j in range(T):
        last = L - T + j
        outs.append(brute_decode(qs[j], K_log[:last + 1], V_log[:last + 1], scale)[0])
    return outs


@pytest.mark.parametrize("seed", [0, 1])
def test_multi_query_matches_causal_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, T, Hkv, G, D, PS = 3, 4, 2, 2, 8, 4
    lens = [5, 9, 4]
    rows_k = [rng.standard_normal((L, Hkv, D)) for L in lens]
    rows_v = [rng.standard_normal((L, Hkv, D)) for L in lens]
    pk, table = scatter_to_pool(rows_k, PS, 12, np.random.default_rng(seed + 7))
    pv = np.full_like(pk, np.nan)
    for b in range(B):
        for i, page in enumerate(table[b]):
            if page >= 0:
                chunk = rows_v[b][i * PS:(i + 1) * PS]
                pv[page, :len(chunk)] = chunk
    q = rng.standard_normal((B, T, Hkv * G, D)).astype(np.float32)
    out, lse = O.paged_multi_query_attention(q, pk.astype(np.float32), pv.astype(np.float32),
                                             table, np.array(lens), 0.3, "f32")
    for b in range(B):
        ref = brute_causal(q[b].astype(np.float64).tolist(),
                           rows_k[b].astype(np.float32).astype(np.float64).tolist(),
                           rows_v[b].astype(np.float32).astype(np.float64).tolist(),
                           float(np.float32(0.3)))
        assert np.abs(out[b] - np.array(ref)).max() < 1e-12


def test_multi_query_is_causal_and_last_query_is_the_decode():
    rng = np.random.default_rng(3)
    B, T, Hkv, G, D, PS = 2, 3, 1, 4, 16, 4
    lens = np.array([10, 7])
    rows_k = [rng.standard_normal((L, Hkv, D)) for L in lens]
    rows_v = [rng.standard_normal((L, Hkv, D)) for L in lens]
    pk, table = scatter_to_pool(rows_k, PS, 8, np.random.default_rng(1))
    pv, _ = scatter_to_pool(rows_v, PS, 8, np.random.default_rng(1))
    q = rng.standard_normal((B, T, G, D))
    out, _ = O.paged_multi_query_attention(q, pk, pv, table, lens, 0.25, "f32")
    full, _ = O.paged_decode_attention(np.ascontiguousarray(q[:, -1]), pk, pv, table, lens, 0.25, "f32")
    assert np.abs(out[:, -1] - full).max() < 1e-13
    # changing the last token's key moves only the last query of that sequence
    pk2 = pk.copy()
    b, L = 0, int(lens[0])
    pk2[table[b, (L - 1) // PS], (L - 1) % PS] += 3.0
    out2, _ = O.paged_multi_query_attention(q, pk2, pv, table, lens, 0.25, "f32")
    assert np.array_equal(out2[0, :-1], out[0, :-1]) and np.array_equal(out2[1], out[1])
    assert np.abs(out2[0, -1] - out[0, -1]).max() > 1e-6
    # a sequence shorter than T: its first queries see nothing
    out3, lse3 = O.paged_multi_query_attention(q, pk, pv, table, np.array([2, 7]), 0.25, "f32")
    assert np.all(out3[0, 0] == 0) and np.all(np.isneginf(lse3[0, 0]))
    assert np.isfinite(lse3[0, 1:]).all()
