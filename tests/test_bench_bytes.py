"""The algorithmic bytes bench.py divides by (the roofline's numerator), recounted here one
sequence at a time from the workload itself: every live token's K and V rows once, q and out,
the page ids the sequence uses and its length, the appended rows (read and written), and, for the
fixed-partition paths, each partition's partial row written and read back."""
import numpy as np
import pytest

import bench
import workloads as W


def recount(w, path, P=None, T=1):
    cfg = w.cfg
    e, Hq, Hkv, D, PS = cfg.elem_bytes, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    kv = q = out = table = append = partials = 0
    for L in w.context_lens.tolist():
        L = max(int(L), 0)
        kv += L * Hkv * D * e * 2
        q += T * Hq * D * e
        out += T * Hq * D * e
        table += ((L + PS - 1) // PS) * 4 + 4
        append += 2 * (2 * Hkv * D * e)
        if path == "split":
            partials += ((L + P - 1) // P) * Hq * (D + 1) * 4
        elif path == "multiquery":
            for j in range(T):
                Lj = max(L - T + 1 + j, 0)
                partials += ((Lj + P - 1) // P) * Hq * (D + 1) * 4
    return dict(kv=kv, q=q, out=out, table=table, append=append, partials=partials)


@pytest.fixture(scope="module")
def qwen():
    w = W.make_workload(W.config(4))
    w.q_tokens = 1
    return w


def test_step_bytes_recount(qwen):
    c = recount(qwen, "step")
    got = bench.step_bytes(qwen, 512, "step")
    assert got["kv"] == c["kv"]
    assert got["kernel"] == got["step"] == c["kv"] + c["q"] + c["out"] + c["table"] + c["append"]


def test_split_bytes_recount(qwen):
    c = recount(qwen, "split", P=512)
    got = bench.step_bytes(qwen, 512, "split")
    assert got["kernel"] == c["kv"] + c["q"] + c["table"] + c["partials"]
    # the merge reads the partials back and reads the lengths again
    assert got["step"] == (c["kv"] + c["q"] + c["out"] + c["table"] + c["append"] + 2 * c["partials"]
                           + len(qwen.context_lens) * 4)


@pytest.mark.parametrize("T", [1, 8])
def test_multi_query_bytes_recount(qwen, T):
    qwen.q_tokens = T
    try:
        c = recount(qwen, "multiquery", P=1024, T=T)
        got = bench.step_bytes(qwen, 1024, "multiquery")
        assert got["kernel"] == c["kv"] + c["q"] + c["table"] + c["partials"]
        got_s = bench.step_bytes(qwen, 1024, "multiquery-step")
        # one launch, no append, no partials counted: K/V once for all T queries
        assert got_s["kernel"] == got_s["step"] == c["kv"] + c["q"] + c["out"] + c["table"]
    finally:
        qwen.q_tokens = 1


def test_headline_bytes_per_step():
    """The Llama-3-8B-shaped batch (64 sequences, contexts U[512, 4096], seed 2): 152,494 live
    tokens of 8 KV heads x 128 dims x 2 bytes x (K, V), plus q, out, page ids, lengths and the
    appended rows."""
    w = W.make_workload(W.config(2))
    w.q_tokens = 1
    assert int(w.context_lens.sum()) == 152494
    got = bench.step_bytes(w, 512, "step")
    assert got["kv"] == 152494 * 8 * 128 * 2 * 2 == 624615424
    assert got["step"] == 626226784
