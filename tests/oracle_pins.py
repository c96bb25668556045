"""Pins of the CPU oracle against facts that do not come from the oracle.

Each ``check_*`` takes the oracle module (``oracle.paged_attention`` or a
mutant of it) and raises ``AssertionError`` when the oracle disagrees with:

* hand-derived golden fixtures under ``tests/golden`` (closed forms);
* brute force: pure-Python loops with ``math.exp``/``math.fsum`` over the
  *logical* history built straight from the inputs, never through a pool;
* invariants the method fixes: paged read == gather, permuting physical
  blocks changes nothing, GQA == MHA over ``np.repeat``-ed KV heads, batched
  == one sequence at a time, poison past the context is never read,
  copy-on-write sharing == deep copies, the partition/LSE merge == the plain
  softmax, prefill row ``i`` == decode at context ``i+1`` and causality;
* closed forms: context 1 gives ``V[0]`` exactly, ``q = 0`` gives the mean of
  ``V``, equal keys give the mean, a dominant key gives its value row,
  linearity in ``V``, invariance to a common key shift, no overflow at large
  scores.

The same checks run against deliberately broken copies of the oracle in
``test_oracle_mutants.py`` to show that plausible mistakes are caught.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# small builders that do not use the oracle
# ---------------------------------------------------------------------------

def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _scatter_logical(orc, hist_k, hist_v, tables, block_size, num_blocks, dtype=np.float32,
                     fill=np.nan):
    """Pools holding each sequence's logical history, written with the
    oracle's slot mapping + write (these are the paths under test)."""
    S = len(hist_k)
    Hkv, D = hist_k[0].shape[1:]
    k_cache = np.full((num_blocks, block_size, Hkv, D), fill, dtype=dtype)
    v_cache = np.full_like(k_cache, fill)
    lens = np.array([h.shape[0] for h in hist_k], dtype=np.int32)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = orc.slot_mapping(tables, lens, block_size, q_start_loc=qsl)
    if lens.sum():
        orc.write_kv_cache(k_cache, v_cache, np.concatenate(hist_k), np.concatenate(hist_v), slots)
    return k_cache, v_cache, lens


def _random_tables(rng, lens, block_size, num_blocks, width=None):
    nblk = [-(-int(L) // block_size) for L in lens]
    width = width or max(max(nblk), 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    pad = perm[-1]
    t = np.full((len(lens), width), pad, dtype=np.int32)
    c = 0
    for s, nb in enumerate(nblk):
        t[s, :nb] = perm[c:c + nb]
        c += nb
    return t


def brute_force_attention(q, keys, values, scale):
    """Textbook softmax attention in pure Python: weights exp(z_t - max z)
    normalised by their exactly rounded sum (math.fsum)."""
    n = len(keys)
    D = len(values[0]) if n else len(q)
    if n == 0:
        return [0.0] * D
    z = [scale * math.fsum(float(q[d]) * float(keys[t][d]) for d in range(len(q))) for t in range(n)]
    zmax = max(z)
    e = [math.exp(x - zmax) for x in z]
    tot = math.fsum(e)
    return [math.fsum(e[t] * float(values[t][d]) for t in range(n)) / tot for d in range(D)]


# ---------------------------------------------------------------------------
# golden fixtures
# ---------------------------------------------------------------------------

def check_golden_slots(orc):
    g = _load("slot_mapping_b4.json")
    B = g["block_size"]
    tables = np.array(g["block_tables"], dtype=np.int32)
    lens = np.array(g["context_lens"], dtype=np.int32)
    got = orc.slot_mapping(tables, lens, B)
    assert got.dtype == np.int64
    assert got.tolist() == g["decode_slots"], got
    got = orc.slot_mapping(tables, lens, B, q_start_loc=np.array(g["prefill_q_start_loc"]))
    assert got.tolist() == g["prefill_slots"], got
    got = orc.slot_mapping(np.array(g["short_block_tables"], dtype=np.int32),
                           np.array(g["short_context_lens"]), B,
                           q_start_loc=np.array(g["short_q_start_loc"]))
    assert got.tolist() == g["short_slots"], got


def _golden_pool(orc, g):
    B, N = g["block_size"], g["num_blocks"]
    keys = np.array(g["keys"], dtype=np.float32)
    vals = np.array(g["values"], dtype=np.float32)
    table = np.array([g["block_table"]], dtype=np.int32)
    k_cache, v_cache, lens = _scatter_logical(orc, [keys[:, None, :]], [vals[:, None, :]],
                                              table, B, N)
    return k_cache, v_cache, table, lens


def check_golden_attention(orc):
    g = _load("attention_closed_form.json")
    tol = g["tolerance"]
    k_cache, v_cache, table, lens = _golden_pool(orc, g)
    q = np.array(g["q_heads"], dtype=np.float32)[None]          # [1, 2, 2]
    out = orc.decode(q, k_cache, v_cache, table, lens, 1.0, orc.F32)
    assert np.max(np.abs(out[0] - np.array(g["decode_expected"]))) < tol, out
    # causal prefill of the three positions, head 0 only carries the checked query
    qp = np.zeros((3, 2, 2), dtype=np.float32)
    qp[:, 0, :] = np.array(g["prefill_q"], dtype=np.float32)
    out = orc.prefill(qp, k_cache, v_cache, table, lens, np.array([0, 3]), 1.0, orc.F32)
    assert np.max(np.abs(out[:, 0, :] - np.array(g["prefill_expected_head0"]))) < tol, out
    # four new tokens over the three-token context: the oldest has no position
    qs = np.zeros((4, 2, 2), dtype=np.float32)
    qs[:, 0, :] = np.array(g["short_prefill_q"], dtype=np.float32)
    out = orc.prefill(qs, k_cache, v_cache, table, lens, np.array([0, 4]), 1.0, orc.F32)
    assert np.all(np.isfinite(out)), out
    assert np.max(np.abs(out[:, 0, :] - np.array(g["short_prefill_expected_head0"]))) < tol, out
    # context length 1 reads v0 exactly
    out = orc.decode(q, k_cache, v_cache, table, np.array([1]), 1.0, orc.F32)
    assert np.array_equal(out[0, 0], np.array(g["values"][0])), out
    # merge of two one-token partitions
    got = orc.lse_merge(np.array(g["merge_m"]), np.array(g["merge_l"]), np.array(g["merge_o"]))
    assert np.max(np.abs(got - np.array(g["merge_expected"]))) < tol, got


def check_bf16_constants(orc):
    g = _load("bf16_values.json")
    got = orc.bf16_bits_to_f64(np.array(g["bits"], dtype=np.uint16))
    want = [eval(r, {"inf": math.inf}) for r in g["values_repr"]]   # noqa: S307 (fixture literals)
    for a, b in zip(got.tolist(), want):
        assert a == b and math.copysign(1.0, a) == math.copysign(1.0, b), (got, want)


# ---------------------------------------------------------------------------
# write / read paths
# ---------------------------------------------------------------------------

def check_write_roundtrip(orc):
    rng = _rng(11)
    B, N, Hkv, D = 4, 23, 2, 3
    lens = [9, 4, 13, 1]
    tables = _random_tables(rng, lens, B, N)
    hist_k = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    hist_v = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    k_cache, v_cache, lens_a = _scatter_logical(orc, hist_k, hist_v, tables, B, N)
    for s, L in enumerate(lens):
        gk = orc.gather_history(k_cache, tables[s], L)
        gv = orc.gather_history(v_cache, tables[s], L)
        assert gk.tobytes() == hist_k[s].tobytes() and gv.tobytes() == hist_v[s].tobytes()
    # every written token landed in its own row and nothing else was touched
    for cache in (k_cache, v_cache):
        touched = ~np.all(np.isnan(cache.reshape(N * B, -1)), axis=1)
        assert int(touched.sum()) == sum(lens)
    # negative slots are skipped; everything else is a verbatim copy
    before = k_cache.copy()
    orc.write_kv_cache(k_cache, v_cache, np.ones((2, Hkv, D), np.float32),
                       np.ones((2, Hkv, D), np.float32), np.array([-1, -5]))
    assert before.tobytes() == k_cache.tobytes()
    # bf16 bit patterns are copied unchanged
    kb = np.zeros((N, B, Hkv, D), np.uint16)
    vb = np.zeros_like(kb)
    pat = rng.integers(0, 65536, size=(3, Hkv, D), dtype=np.uint16)
    orc.write_kv_cache(kb, vb, pat, pat[::-1].copy(), np.array([5, 17, 40]))
    assert kb.reshape(N * B, Hkv, D)[[5, 17, 40]].tobytes() == pat.tobytes()
    assert vb.reshape(N * B, Hkv, D)[[5, 17, 40]].tobytes() == pat[::-1].tobytes()


def check_gather_equals_paged_read(orc):
    rng = _rng(12)
    B, N, Hkv, D = 16, 40, 3, 5
    lens = [1, 16, 17, 45, 0]
    tables = _random_tables(rng, lens, B, N)
    hist = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    k_cache, _, _ = _scatter_logical(orc, hist, hist, tables, B, N)
    for s, L in enumerate(lens):
        a = orc.gather_history(k_cache, tables[s], L)
        b = orc.read_through_table(k_cache, tables[s], L)
        assert a.shape == (L, Hkv, D) and a.tobytes() == b.tobytes()


# ---------------------------------------------------------------------------
# attention against brute force
# ---------------------------------------------------------------------------

def _decode_case(orc, rng, lens, Hq, Hkv, D, B, N, scale, tables=None):
    tables = _random_tables(rng, lens, B, N) if tables is None else tables
    hist_k = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    hist_v = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    k_cache, v_cache, lens_a = _scatter_logical(orc, hist_k, hist_v, tables, B, N)
    out = orc.decode(q, k_cache, v_cache, tables, lens_a, scale, orc.F32)
    return q, hist_k, hist_v, out


def check_brute_force_decode(orc):
    rng = _rng(13)
    for (lens, Hq, Hkv, D, B) in [([5, 1, 13], 4, 2, 3, 4), ([48], 2, 1, 8, 16),
                                  ([7, 0, 16, 17], 6, 3, 2, 8)]:
        scale = 0.37
        q, hk, hv, out = _decode_case(orc, rng, lens, Hq, Hkv, D, B, 64, scale)
        n_rep = Hq // Hkv
        for s, L in enumerate(lens):
            for h in range(Hq):
                g = h // n_rep
                want = brute_force_attention(q[s, h], hk[s][:, g].tolist(), hv[s][:, g].tolist(),
                                             scale)
                assert np.max(np.abs(out[s, h] - np.array(want))) < 1e-12, (lens, s, h)
    # every ordering of a 4-block table gives the same output, bitwise
    B, lens = 4, [15]
    base = None
    hk = [rng.standard_normal((15, 1, 4)).astype(np.float32)]
    hv = [rng.standard_normal((15, 1, 4)).astype(np.float32)]
    q = rng.standard_normal((1, 1, 4)).astype(np.float32)
    want = brute_force_attention(q[0, 0], hk[0][:, 0].tolist(), hv[0][:, 0].tolist(), 0.5)
    for perm in itertools.permutations([2, 5, 7, 9]):
        tables = np.array([list(perm) + [0]], dtype=np.int32)
        k_cache, v_cache, la = _scatter_logical(orc, hk, hv, tables, B, 10)
        out = orc.decode(q, k_cache, v_cache, tables, la, 0.5, orc.F32)
        if base is None:
            base = out
            assert np.max(np.abs(out[0, 0] - np.array(want))) < 1e-12
        assert out.tobytes() == base.tobytes(), perm


def check_brute_force_prefill(orc):
    rng = _rng(14)
    B, N, Hq, Hkv, D, scale = 4, 32, 4, 2, 3, 0.8
    ctx = [9, 6, 12]
    qlen = [9, 2, 5]              # full prompt, short continuation, mid continuation
    tables = _random_tables(rng, ctx, B, N)
    hk = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in ctx]
    hv = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in ctx]
    k_cache, v_cache, la = _scatter_logical(orc, hk, hv, tables, B, N)
    qsl = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32)
    out = orc.prefill(q, k_cache, v_cache, tables, la, qsl, scale, orc.F32)
    n_rep = Hq // Hkv
    for s in range(len(ctx)):
        for i in range(qlen[s]):
            t = int(qsl[s]) + i
            pos = ctx[s] - qlen[s] + i
            for h in range(Hq):
                g = h // n_rep
                want = brute_force_attention(q[t, h], hk[s][:pos + 1, g].tolist(),
                                             hv[s][:pos + 1, g].tolist(), scale)
                assert np.max(np.abs(out[t, h] - np.array(want))) < 1e-12, (s, i, h)


def check_brute_force_prefill_short_context(orc):
    """More new tokens than the context holds: a token whose position
    (context length - q_len + i) is negative sees no key and gives zeros;
    every other row is brute-force attention over positions 0..p.  An empty
    context gives zeros for all its tokens.  GQA groups of 3, ragged tables."""
    rng = _rng(22)
    B, N, Hq, Hkv, D, scale = 4, 32, 6, 2, 3, 0.6
    ctx = [5, 0, 9, 3]
    qlen = [8, 2, 9, 1]           # longer than the context, empty context, whole, decode
    tables = _random_tables(rng, [max(L, 1) for L in ctx], B, N)
    hk = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in ctx]
    hv = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in ctx]
    k_cache, v_cache, la = _scatter_logical(orc, hk, hv, tables, B, N)
    qsl = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32)
    out = orc.prefill(q, k_cache, v_cache, tables, la, qsl, scale, orc.F32)
    assert np.all(np.isfinite(out))
    n_rep = Hq // Hkv
    for s in range(len(ctx)):
        for i in range(qlen[s]):
            t = int(qsl[s]) + i
            pos = ctx[s] - qlen[s] + i
            for h in range(Hq):
                g = h // n_rep
                if pos < 0:
                    assert np.array_equal(out[t, h], np.zeros(D)), (s, i, h)
                    continue
                want = brute_force_attention(q[t, h], hk[s][:pos + 1, g].tolist(),
                                             hv[s][:pos + 1, g].tolist(), scale)
                assert np.max(np.abs(out[t, h] - np.array(want))) < 1e-12, (s, i, h)
    # scores in the thousands: finite, and the brute-force value
    big = (q * 1000).astype(np.float32)
    out = orc.prefill(big, k_cache, v_cache, tables, la, qsl, 1.0, orc.F32)
    assert np.all(np.isfinite(out))
    s, i, h = 2, 8, 5
    t, g = int(qsl[s]) + i, h // n_rep
    want = brute_force_attention(big[t, h], hk[s][:, g].tolist(), hv[s][:, g].tolist(), 1.0)
    assert np.max(np.abs(out[t, h] - np.array(want))) < 1e-9


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def check_closed_forms(orc):
    rng = _rng(15)
    B, N, Hq, Hkv, D = 4, 24, 2, 1, 6
    L = 11
    tables = _random_tables(rng, [L], B, N)
    hk = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    hv = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)

    def run(k, v, qq, scale=0.4, lens=None):
        kc, vc, la = _scatter_logical(orc, [k], [v], tables, B, N)
        return orc.decode(qq, kc, vc, tables, la if lens is None else np.array(lens), scale,
                          orc.F32)

    # context length 1 reads V[0] exactly, whatever the query
    out = run(hk, hv, q, lens=[1])
    assert np.array_equal(out[0, 0], hv[0, 0].astype(np.float64))
    # zero query: uniform weights -> mean of V
    out = run(hk, hv, np.zeros_like(q))
    assert np.max(np.abs(out[0, 0] - hv[:, 0].astype(np.float64).mean(0))) < 1e-12
    # equal keys: uniform weights -> mean of V
    out = run(np.repeat(hk[:1], L, 0), hv, q)
    assert np.max(np.abs(out[0, 1] - hv[:, 0].astype(np.float64).mean(0))) < 1e-12
    # one key far ahead of the rest (score gap >= 50): its value row
    k2 = (0.01 * hk).astype(np.float32)
    k2[7, 0] = (q[0, 0] / np.linalg.norm(q[0, 0]) * 400).astype(np.float32)
    out = run(k2, hv, q, scale=1.0)
    assert np.max(np.abs(out[0, 0] - hv[7, 0])) < 1e-9
    # linear in V: V*c -> out*c, V + c -> out + c
    base = run(hk, hv, q)
    out = run(hk, (hv * 4).astype(np.float32), q)
    assert np.max(np.abs(out - 4 * base)) < 1e-12
    shift = rng.standard_normal(D).astype(np.float32)
    out = run(hk, (hv.astype(np.float64) + shift).astype(np.float32), q)
    exact_shifted = run(hk, hv, q) + shift.astype(np.float64)
    assert np.max(np.abs(out - exact_shifted)) < 1e-6       # float32 storage of v+shift
    # a shift common to every key changes every score of a head by one constant
    w = np.zeros(D, np.float32)
    w[0] = 1.5
    out = run((hk + w).astype(np.float32), hv, q)
    assert np.max(np.abs(out - base)) < 1e-6
    # large scores: no overflow, and the brute-force value
    out = run(hk, hv, (q * 300).astype(np.float32), scale=1.0)
    want = brute_force_attention((q[0, 0] * 300).astype(np.float32), hk[:, 0].tolist(),
                                 hv[:, 0].tolist(), 1.0)
    assert np.all(np.isfinite(out)) and np.max(np.abs(out[0, 0] - np.array(want))) < 1e-9


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def check_gqa_equals_repeated_mha(orc):
    rng = _rng(16)
    B, N, Hq, Hkv, D = 4, 64, 8, 2, 5
    lens = [10, 21]
    tables = _random_tables(rng, lens, B, N)
    hk = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    hv = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    kc, vc, la = _scatter_logical(orc, hk, hv, tables, B, N)
    gqa = orc.decode(q, kc, vc, tables, la, 0.3, orc.F32)
    rk = [np.repeat(x, Hq // Hkv, axis=1) for x in hk]
    rv = [np.repeat(x, Hq // Hkv, axis=1) for x in hv]
    kc2, vc2, _ = _scatter_logical(orc, rk, rv, tables, B, N)
    mha = orc.decode(q, kc2, vc2, tables, la, 0.3, orc.F32)
    assert np.max(np.abs(gqa - mha)) < 1e-13


def check_variable_lengths(orc):
    rng = _rng(17)
    B, N, Hq, Hkv, D = 4, 64, 4, 2, 3
    lens = [3, 17, 1, 8]
    tables = _random_tables(rng, lens, B, N)
    q, hk, hv, out = _decode_case(orc, rng, lens, Hq, Hkv, D, B, N, 0.5, tables=tables)
    for s, L in enumerate(lens):
        kc, vc, la = _scatter_logical(orc, [hk[s]], [hv[s]], tables[s:s + 1], B, N)
        one = orc.decode(q[s:s + 1], kc, vc, tables[s:s + 1], la, 0.5, orc.F32)
        assert one.tobytes() == out[s:s + 1].tobytes()


def check_partial_block_poison(orc):
    rng = _rng(18)
    B, N, Hq, Hkv, D = 8, 16, 2, 2, 4
    lens = [13]
    tables = _random_tables(rng, lens, B, N, width=5)   # 3 unused table entries
    hk = [rng.standard_normal((13, Hkv, D)).astype(np.float32)]
    hv = [rng.standard_normal((13, Hkv, D)).astype(np.float32)]
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    kn, vn, la = _scatter_logical(orc, hk, hv, tables, B, N, fill=np.nan)
    kz, vz, _ = _scatter_logical(orc, hk, hv, tables, B, N, fill=0.0)
    a = orc.decode(q, kn, vn, tables, la, 0.5, orc.F32)
    b = orc.decode(q, kz, vz, tables, la, 0.5, orc.F32)
    assert np.all(np.isfinite(a)) and a.tobytes() == b.tobytes()
    qsl = np.array([0, 13])
    qp = rng.standard_normal((13, Hq, D)).astype(np.float32)
    a = orc.prefill(qp, kn, vn, tables, la, qsl, 0.5, orc.F32)
    b = orc.prefill(qp, kz, vz, tables, la, qsl, 0.5, orc.F32)
    assert np.all(np.isfinite(a)) and a.tobytes() == b.tobytes()


def check_cow_shared_equals_copied(orc):
    rng = _rng(19)
    B, N, Hq, Hkv, D = 4, 64, 4, 2, 3
    prefix_blocks = 3
    lens = [prefix_blocks * B + 5, prefix_blocks * B + 2, prefix_blocks * B + 7]
    perm = rng.permutation(N).astype(np.int32)
    prefix = perm[:prefix_blocks]
    shared = np.zeros((3, 6), np.int32)
    copied = np.zeros((3, 6), np.int32)
    c = prefix_blocks
    for s, L in enumerate(lens):
        own = -(-L // B) - prefix_blocks
        shared[s, :prefix_blocks] = prefix
        shared[s, prefix_blocks:prefix_blocks + own] = perm[c:c + own]
        c += own
    for s, L in enumerate(lens):
        nb = -(-L // B)
        copied[s, :nb] = perm[c:c + nb]
        c += nb
    pk = rng.standard_normal((prefix_blocks * B, Hkv, D)).astype(np.float32)
    pv = rng.standard_normal((prefix_blocks * B, Hkv, D)).astype(np.float32)
    sk = [rng.standard_normal((L - prefix_blocks * B, Hkv, D)).astype(np.float32) for L in lens]
    sv = [rng.standard_normal((L - prefix_blocks * B, Hkv, D)).astype(np.float32) for L in lens]
    hk = [np.concatenate([pk, x]) for x in sk]
    hv = [np.concatenate([pv, x]) for x in sv]
    q = rng.standard_normal((3, Hq, D)).astype(np.float32)
    # shared: prefix rows written once (by sequence 0), suffixes by each sequence
    kc = np.full((N, B, Hkv, D), np.nan, np.float32)
    vc = np.full_like(kc, np.nan)
    slots = orc.slot_mapping(shared[:1], [prefix_blocks * B], B,
                             q_start_loc=np.array([0, prefix_blocks * B]))
    orc.write_kv_cache(kc, vc, pk, pv, slots)
    qsl = np.concatenate([[0], np.cumsum([x.shape[0] for x in sk])])
    slots = orc.slot_mapping(shared, lens, B, q_start_loc=qsl)
    orc.write_kv_cache(kc, vc, np.concatenate(sk), np.concatenate(sv), slots)
    a = orc.decode(q, kc, vc, shared, np.array(lens), 0.6, orc.F32)
    kc2, vc2, la = _scatter_logical(orc, hk, hv, copied, B, N)
    b = orc.decode(q, kc2, vc2, copied, la, 0.6, orc.F32)
    assert a.tobytes() == b.tobytes()


def check_partition_merge(orc):
    rng = _rng(20)
    D = 6
    for n in [1, 5, 16, 37]:
        k = rng.standard_normal((n, D))
        v = rng.standard_normal((n, D))
        q = rng.standard_normal(D) * 2
        want = brute_force_attention(q, k.tolist(), v.tolist(), 0.7)
        for P in [1, 3, 16, 64]:
            m, l, o = orc.partition_stats(q, k, v, 0.7, P)
            assert m.shape[0] == -(-n // P)
            got = orc.lse_merge(m, l, o)
            assert np.max(np.abs(got - np.array(want))) < 1e-12, (n, P)
    assert np.array_equal(orc.lse_merge(np.zeros(0), np.zeros(0), np.zeros((0, D))), np.zeros(D))


def check_prefill_rows_equal_decode(orc):
    rng = _rng(21)
    B, N, Hq, Hkv, D = 4, 40, 4, 1, 5
    L = 14
    tables = _random_tables(rng, [L], B, N)
    hk = [rng.standard_normal((L, Hkv, D)).astype(np.float32)]
    hv = [rng.standard_normal((L, Hkv, D)).astype(np.float32)]
    kc, vc, la = _scatter_logical(orc, hk, hv, tables, B, N)
    q = rng.standard_normal((L, Hq, D)).astype(np.float32)
    qsl = np.array([0, L])
    out = orc.prefill(q, kc, vc, tables, la, qsl, 0.45, orc.F32)
    for i in range(L):
        d = orc.decode(q[i:i + 1], kc, vc, tables, np.array([i + 1]), 0.45, orc.F32)
        assert np.max(np.abs(out[i] - d[0])) < 1e-13, i
    # causality: changing K/V after position i leaves row i bitwise unchanged
    i = 6
    hk2 = [hk[0].copy()]
    hv2 = [hv[0].copy()]
    hk2[0][i + 1:] += 3.0
    hv2[0][i + 1:] -= 2.0
    kc2, vc2, _ = _scatter_logical(orc, hk2, hv2, tables, B, N)
    out2 = orc.prefill(q, kc2, vc2, tables, la, qsl, 0.45, orc.F32)
    assert out2[:i + 1].tobytes() == out[:i + 1].tobytes()
    assert not np.array_equal(out2[i + 1:], out[i + 1:])


ALL_CHECKS = [
    check_golden_slots, check_golden_attention, check_bf16_constants, check_write_roundtrip,
    check_gather_equals_paged_read, check_brute_force_decode, check_brute_force_prefill,
    check_brute_force_prefill_short_context,
    check_closed_forms, check_gqa_equals_repeated_mha, check_variable_lengths,
    check_partial_block_poison, check_cow_shared_equals_copied, check_partition_merge,
    check_prefill_rows_equal_decode,
]
