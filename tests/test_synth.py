"""The seeded input generator: determinism, thread independence, moments,
and the needle construction."""
import math

import numpy as np

import hils_synth as hs


def test_deterministic_and_thread_independent():
    a = hs.normal((100001,), 7, 3, 1.0, dtype="f32", nthreads=1)
    b = hs.normal((100001,), 7, 3, 1.0, dtype="f32", nthreads=7)
    c = hs.normal((100001,), 7, 3, 1.0, dtype="f32", nthreads=16)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    u1 = hs.uniform((5003,), 1, 2, 0.0, 1.0, dtype="f64", nthreads=1)
    u2 = hs.uniform((5003,), 1, 2, 0.0, 1.0, dtype="f64", nthreads=5)
    assert np.array_equal(u1, u2)


def test_prefix_stability():
    """Element i does not depend on the array length."""
    a = hs.normal((1000,), 3, 1, dtype="f64")
    b = hs.normal((1001,), 3, 1, dtype="f64")
    assert np.array_equal(a, b[:1000])


def test_streams_and_seeds_differ():
    a = hs.normal((1000,), 1, 1, dtype="f64")
    assert not np.array_equal(a, hs.normal((1000,), 1, 2, dtype="f64"))
    assert not np.array_equal(a, hs.normal((1000,), 2, 1, dtype="f64"))


def test_moments():
    x = hs.normal((1 << 20,), 11, 1, 2.0, 0.5, dtype="f64")
    assert abs(x.mean() - 0.5) < 0.01 and abs(x.std() - 2.0) < 0.01
    u = hs.uniform((1 << 20,), 11, 2, -1.0, 3.0, dtype="f64")
    assert u.min() >= -1.0 and u.max() < 3.0 and abs(u.mean() - 1.0) < 0.01


def test_bf16_storage_is_the_rounded_f32():
    f = hs.normal((4096,), 5, 1, 3.0, dtype="f32")
    b = hs.normal((4096,), 5, 1, 3.0, dtype="bf16")
    assert np.array_equal(b, hs.f32_to_bf16(f))
    assert np.abs(hs.bf16_to_f32(b) - f).max() <= np.abs(f).max() * 2 ** -8


def test_prefill_needles():
    wl = hs.Workload("t", "prefill", 2, 2048, 8, 2, 64, top_k=4, window=256,
                     qkv_std=0.125, needles="frac:0.1")
    inp = hs.prefill_inputs(wl, 3)
    nd = inp["needles"]
    assert len(nd) == 2 * 2 * round(0.1 * 32)
    for n in nd:
        k = hs.as_f64(inp["k"][n["b"], n["g"], n["pos"]])
        q = hs.as_f64(inp["q"][n["b"], n["h"], n["query"]])
        cos = k @ q / np.linalg.norm(k) / np.linalg.norm(q)
        assert abs(cos - 0.9) < 0.02
        # the target query can select the needle's chunk
        assert (n["query"] - wl.window + 1) // wl.chunk_size > n["chunk"]
        lm = hs.as_f64(inp["q_lm"][n["b"], n["h"], n["chunk"]])
        assert lm @ k / np.linalg.norm(lm) / np.linalg.norm(k) > 0.99


def test_decode_needles_even_depths():
    wl = hs.Workload("t", "decode", 1, 4096, 4, 2, 32, needles="even:10")
    inp = hs.decode_inputs(wl, 1)
    n = (4096 - 1 - 512 + 1) // 64
    chunks = sorted({x["chunk"] for x in inp["needles"]})
    assert chunks == sorted({int(math.floor((k + 0.5) * n / 10)) for k in range(10)})
    assert inp["seq_lens"].tolist() == [4096]


def test_synthetic_summaries_ranges():
    wl = hs.Workload("t", "decode", 2, 1024, 4, 2, 32)
    s = hs.synthetic_summaries(wl, 1)
    assert s["k_sum"].shape == (2, 4, 16, 32) and s["k_sum"].dtype == np.uint16
    assert s["b_sum"].min() >= 0 and s["b_sum"].max() <= math.log(64)
