"""Pins of the CPU oracle against what mathematics and library routines fix.

Each test checks one oracle function against something other than itself: a
closed form, an invariant, a special case that reduces to a library routine
(numpy float64 matmul, torch's bf16 conversion, scipy's logistic), or brute
force on tiny inputs. The cases are chosen so that a plausible slip (a
dropped term, a wrong sign, a transposed operand, a wrong head or page
index) fails at least one of them.
"""
import math
from dataclasses import replace

import numpy as np
import pytest
import scipy.special
import torch

import synthetic
from oracle import dims_of

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf16_to_f64(bits):
    """bf16 pattern -> value, by definition (upper half of a binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def torch_bf16_rne(x):
    """Library bf16 rounding (round to nearest even) of binary32 values."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def small_cfg(**kw):
    base = dict(cid=101, name="pin", n_layers=1, hidden=64, n_q_heads=4, n_kv_heads=2,
                head_dim=16, ffn=96, vocab=50, has_embed=True, batch=1, kv_len=5, steps=1)
    base.update(kw)
    return synthetic.Workload(**base)


# --------------------------------------------------------------------- bf16

def test_bf16_roundtrip_all_patterns(oracle64):
    for h in range(0, 1 << 16, 1):
        f = oracle64.bf16_to_f32(h)
        if math.isnan(f):
            back = oracle64.f32_to_bf16(f)
            assert (back & 0x7f80) == 0x7f80 and (back & 0x7f) != 0
            continue
        assert oracle64.f32_to_bf16(f) == h, hex(h)


def test_bf16_rne_halfway_and_neighbours(oracle64):
    rng = np.random.default_rng(7)
    pats = np.concatenate([np.arange(0, 0x7f7f, 97), rng.integers(0, 0x7f7f, 300), [0, 1, 0x7f7e]])
    for h in pats:
        for sign in (0, 0x8000):
            hh = int(h) | sign
            base = hh << 16
            for low, expect in ((0x7fff, hh), (0x8001, hh + 1)):
                f = np.array([base | low], dtype=np.uint32).view(np.float32)[0]
                assert oracle64.f32_to_bf16(f) == expect
            mid = np.array([base | 0x8000], dtype=np.uint32).view(np.float32)[0]
            even = hh if (hh & 1) == 0 else hh + 1
            assert oracle64.f32_to_bf16(mid) == even


def test_bf16_overflow_and_library_agreement(oracle64):
    big = np.array([0x7f7f7fff, 0x7f7f8000, 0x7f7fffff], dtype=np.uint32).view(np.float32)
    assert [oracle64.f32_to_bf16(f) for f in big] == [0x7f7f, 0x7f80, 0x7f80]
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4000),
                         rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    xs = xs[np.isfinite(xs)]
    ref = torch_bf16_rne(xs)
    got = np.array([oracle64.f32_to_bf16(f) for f in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------- matvec

@pytest.mark.parametrize("prec", ["f64", "f32"])
def test_matvec_exact_on_integers(prec, oracle64, oracle32):
    o = oracle64 if prec == "f64" else oracle32
    rng = np.random.default_rng(3)
    Wi = rng.integers(-4, 5, size=(7, 13))
    xi = rng.integers(-9, 10, size=13)
    Wb = torch_bf16_rne(Wi.astype(np.float32)).reshape(7, 13)
    y = o.matvec(Wb, xi.astype(np.float64))
    assert np.array_equal(y.astype(np.int64), Wi @ xi)


@pytest.mark.parametrize("prec,u", [("f64", 2.0 ** -53), ("f32", 2.0 ** -24)])
@pytest.mark.parametrize("rows,cols", [(5, 256), (3, 2048), (2, 8192)])
def test_matvec_higham_bound(prec, u, rows, cols, oracle64, oracle32):
    o = oracle64 if prec == "f64" else oracle32
    rng = np.random.default_rng(rows * cols)
    Wb = (rng.standard_normal((rows, cols)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = rng.standard_normal(cols)
    if prec == "f32":
        x = x.astype(np.float32).astype(np.float64)
    W = bf16_to_f64(Wb)
    ref = W @ x
    got = o.matvec(Wb, x)
    gamma = cols * u / (1 - cols * u)
    bound = gamma * (np.abs(W) @ np.abs(x)) + 1e-300
    assert np.all(np.abs(got - ref) <= 1.01 * bound + (4 * u * np.abs(ref) if prec == "f32" else 0))


# ------------------------------------------------------------------ rmsnorm

def test_rmsnorm_constant_vector_closed_form(oracle64):
    ones = np.full(64, 0x3F80, dtype=np.uint16)
    for c in (1e-3, 0.5, 1.0, 3.0, -7.25):
        u = oracle64.rmsnorm(np.full(64, c), ones, 1e-5)
        assert np.allclose(u, c / math.sqrt(c * c + 1e-5), rtol=1e-14, atol=0)


def test_rmsnorm_known_vector_and_weight(oracle64):
    w = torch_bf16_rne(np.array([2.0, -0.5], dtype=np.float32))
    u = oracle64.rmsnorm(np.array([3.0, 4.0]), w, 0.0)
    r = math.sqrt(12.5)
    assert np.allclose(u, [2.0 * 3 / r, -0.5 * 4 / r], rtol=1e-15)


def test_rmsnorm_mean_square_and_scale(oracle64):
    rng = np.random.default_rng(5)
    x = rng.standard_normal(2048)
    ones = np.full(2048, 0x3F80, dtype=np.uint16)
    eps = 1e-5
    u = oracle64.rmsnorm(x, ones, eps)
    ms = np.mean(x * x)
    assert math.isclose(np.mean(u * u), ms / (ms + eps), rel_tol=1e-12)
    u0 = oracle64.rmsnorm(x, ones, 0.0)
    assert np.allclose(oracle64.rmsnorm(17.0 * x, ones, 0.0), u0, rtol=1e-13)
    wb = (rng.standard_normal(2048).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.allclose(oracle64.rmsnorm(x, wb, eps), u * bf16_to_f64(wb), rtol=1e-14)


# --------------------------------------------------------------------- RoPE

def test_rope_identity_at_zero_and_norms(oracle64):
    rng = np.random.default_rng(9)
    v = rng.standard_normal(3 * 64)
    assert np.array_equal(oracle64.rope(v, 3, 64, 0, 10000.0), v)
    r = oracle64.rope(v, 3, 64, 777, 10000.0).reshape(3, 64)
    v3 = v.reshape(3, 64)
    pair_in = v3[:, :32] ** 2 + v3[:, 32:] ** 2
    pair_out = r[:, :32] ** 2 + r[:, 32:] ** 2
    assert np.allclose(pair_in, pair_out, rtol=1e-12)


def test_rope_composition_and_relative_property(oracle64):
    rng = np.random.default_rng(10)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    m, n = 37, 1290
    twice = oracle64.rope(oracle64.rope(q, 1, 64, m, 10000.0), 1, 64, n, 10000.0)
    assert np.allclose(twice, oracle64.rope(q, 1, 64, m + n, 10000.0), atol=1e-11)
    lhs = oracle64.rope(q, 1, 64, m + n, 10000.0) @ oracle64.rope(k, 1, 64, n, 10000.0)
    rhs = oracle64.rope(q, 1, 64, m, 10000.0) @ k
    assert math.isclose(lhs, rhs, rel_tol=1e-10, abs_tol=1e-10)


def test_rope_is_complex_rotation_with_rotate_half_pairing(oracle64):
    # d = 2: the pair (0, 1) at frequency 1 is multiplication by e^{i p}.
    for p in (1, 5, 100):
        z = complex(0.3, -1.7) * complex(math.cos(p), math.sin(p))
        assert np.allclose(oracle64.rope(np.array([0.3, -1.7]), 1, 2, p, 10000.0), [z.real, z.imag])
    # d = 4, theta = 100: index 1 pairs with index 3 at frequency 100^(-2/4).
    p = 3
    e1 = oracle64.rope(np.array([0.0, 1.0, 0.0, 0.0]), 1, 4, p, 100.0)
    f = 100.0 ** -0.5
    assert np.allclose(e1, [0.0, math.cos(p * f), 0.0, math.sin(p * f)], atol=1e-15)
    e0 = oracle64.rope(np.array([1.0, 0.0, 0.0, 0.0]), 1, 4, p, 100.0)
    assert np.allclose(e0, [math.cos(p), 0.0, math.sin(p), 0.0], atol=1e-15)


# --------------------------------------------------------------------- SiLU

def test_silu_identities(oracle64):
    assert oracle64.silu(0.0) == 0.0
    assert math.isclose(oracle64.silu(1.0), scipy.special.expit(1.0), rel_tol=1e-15)
    for z in (0.1, 1.3, 4.0, 11.0):
        assert math.isclose(oracle64.silu(z) - oracle64.silu(-z), z, rel_tol=1e-13)
        assert math.isclose(oracle64.silu(z), z * scipy.special.expit(z), rel_tol=1e-14)
    assert math.isclose(oracle64.silu(60.0), 60.0, rel_tol=1e-15)
    assert abs(oracle64.silu(-60.0)) < 1e-24


# ------------------------------------------------------------------- argmax

def test_argmax_ties_and_library(oracle64):
    v = np.array([0.5, 2.0, -1.0, 2.0, 2.0])
    assert oracle64.argmax(v) == 1
    rng = np.random.default_rng(12)
    for _ in range(50):
        v = rng.integers(-3, 4, size=40).astype(np.float64)
        assert oracle64.argmax(v) == int(np.argmax(v.astype(np.float32)))
    # the decision is taken on binary32 values: these two collapse to a tie
    v = np.array([1.0, 1.0 + 1e-12])
    assert oracle64.argmax(v) == 0
    v[0] = np.nan
    assert oracle64.argmax(v) == -1


# ---------------------------------------------------------------- attention

def _attn_setup(pos, nq=4, nkv=2, d=8, T=4, seed=0, page_perm=None):
    cfg = small_cfg(n_q_heads=nq, n_kv_heads=nkv, head_dim=d, page_tokens=T)
    n_pages = pos // T + 1
    perm = np.arange(n_pages, dtype=np.int32) if page_perm is None else page_perm
    st = synthetic.State(1, np.zeros(1, np.int32), np.array([pos], np.int32),
                         np.zeros((1, n_pages, nkv, T, d), np.uint16),
                         np.zeros((1, n_pages, nkv, T, d), np.uint16),
                         perm[None, :].copy(), n_pages, None)
    rng = np.random.default_rng(seed)
    return cfg, st, rng


def _put(pool, perm, T, j, g, vals):
    pool[0, perm[j // T], g, j % T, :] = torch_bf16_rne(vals)


def test_attention_single_position_returns_v(oracle64):
    cfg, st, rng = _attn_setup(0)
    perm = st.page_table[0]
    vrows = [rng.standard_normal(8) for _ in range(2)]
    for g in range(2):
        _put(st.k_pool, perm, 4, 0, g, rng.standard_normal(8))
        _put(st.v_pool, perm, 4, 0, g, vrows[g])
    q = rng.standard_normal(4 * 8)
    out = oracle64.attention(dims_of(cfg, st), q, st.k_pool[0], st.v_pool[0], perm, 0).reshape(4, 8)
    for h in range(4):
        assert np.array_equal(out[h], bf16_to_f64(st.v_pool[0, perm[0], h // 2, 0]))


def test_attention_equal_keys_give_mean_of_v_and_gqa_grouping(oracle64):
    pos = 9
    cfg, st, rng = _attn_setup(pos, page_perm=np.array([2, 0, 1], np.int32))
    perm = st.page_table[0]
    key = rng.standard_normal(8)
    for j in range(pos + 1):
        for g in range(2):
            _put(st.k_pool, perm, 4, j, g, key)
            _put(st.v_pool, perm, 4, j, g, rng.standard_normal(8) + 10.0 * g)
    q = rng.standard_normal(32)
    out = oracle64.attention(dims_of(cfg, st), q, st.k_pool[0], st.v_pool[0], perm, pos).reshape(4, 8)
    for h in range(4):
        g = h // 2  # contiguous groups of nq / nkv query heads
        rows = np.stack([bf16_to_f64(st.v_pool[0, perm[j // 4], g, j % 4]) for j in range(pos + 1)])
        assert np.allclose(out[h], rows.mean(axis=0), rtol=1e-12, atol=1e-12)


def test_attention_two_positions_logistic_weights(oracle64):
    cfg, st, rng = _attn_setup(1, nq=1, nkv=1)
    perm = st.page_table[0]
    d = 8
    k0, k1 = np.zeros(d), np.zeros(d)
    k0[0] = 1.0
    k1[1] = 1.0
    _put(st.k_pool, perm, 4, 0, 0, k0)
    _put(st.k_pool, perm, 4, 1, 0, k1)
    v0, v1 = rng.standard_normal(d), rng.standard_normal(d)
    _put(st.v_pool, perm, 4, 0, 0, v0)
    _put(st.v_pool, perm, 4, 1, 0, v1)
    q = np.zeros(d)
    q[0], q[1] = 3.0, -2.0
    out = oracle64.attention(dims_of(cfg, st), q, st.k_pool[0], st.v_pool[0], perm, 1)
    w0 = scipy.special.expit((3.0 - (-2.0)) / math.sqrt(d))
    V0, V1 = bf16_to_f64(st.v_pool[0, 0, 0, 0]), bf16_to_f64(st.v_pool[0, 0, 0, 1])
    assert np.allclose(out, w0 * V0 + (1 - w0) * V1, rtol=1e-13)


def test_attention_dominant_key_and_score_shift(oracle64):
    pos = 6
    cfg, st, rng = _attn_setup(pos, nq=2, nkv=1)
    perm = st.page_table[0]
    keys = [rng.standard_normal(8) for _ in range(pos + 1)]
    for j in range(pos + 1):
        _put(st.k_pool, perm, 4, j, 0, keys[j])
        _put(st.v_pool, perm, 4, j, 0, rng.standard_normal(8))
    K = np.stack([bf16_to_f64(st.k_pool[0, perm[j // 4], 0, j % 4]) for j in range(pos + 1)])
    q = np.concatenate([400.0 * rng.standard_normal(8), rng.standard_normal(8)])
    out = oracle64.attention(dims_of(cfg, st), q, st.k_pool[0], st.v_pool[0], perm, pos).reshape(2, 8)
    # head 0: one score dominates (gap checked) -> that V row
    scores = np.sort(K @ q[:8] / math.sqrt(8))
    assert scores[-1] - scores[-2] > 60.0
    top = int(np.argmax(K @ q[:8]))
    assert np.allclose(out[0], bf16_to_f64(st.v_pool[0, perm[top // 4], 0, top % 4]), atol=1e-12)
    # adding the same vector orthogonal to q to every key leaves the output
    cfg2, st2, _ = _attn_setup(pos, nq=2, nkv=1)
    st2.v_pool[:] = st.v_pool
    shift = np.zeros(8)
    shift[7] = 0.5
    q2 = np.concatenate([q[:8], q[8:]])
    q2[7] = 0.0
    q2[15] = 0.0
    for j in range(pos + 1):
        _put(st2.k_pool, perm, 4, j, 0, K[j].copy())
    st_shift = st2.k_pool.copy()
    for j in range(pos + 1):
        st_shift[0, perm[j // 4], 0, j % 4] = torch_bf16_rne(K[j] + shift)
    a = oracle64.attention(dims_of(cfg2, st2), q2, st2.k_pool[0], st2.v_pool[0], perm, pos)
    b = oracle64.attention(dims_of(cfg2, st2), q2, st_shift[0], st2.v_pool[0], perm, pos)
    exact_shift = np.all(torch_bf16_rne(np.stack(K)[:, 7] + 0.5) == torch_bf16_rne(np.stack(K)[:, 7] + 0.5))
    assert exact_shift
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_attention_paged_equals_contiguous(oracle64):
    pos = 13
    perm = np.array([3, 1, 0, 2], np.int32)
    cfg, st, rng = _attn_setup(pos, page_perm=perm)
    cfgc, stc, _ = _attn_setup(pos)
    for j in range(pos + 1):
        for g in range(2):
            kv = rng.standard_normal(8), rng.standard_normal(8)
            _put(st.k_pool, perm, 4, j, g, kv[0])
            _put(st.v_pool, perm, 4, j, g, kv[1])
            _put(stc.k_pool, stc.page_table[0], 4, j, g, kv[0])
            _put(stc.v_pool, stc.page_table[0], 4, j, g, kv[1])
    q = rng.standard_normal(32)
    a = oracle64.attention(dims_of(cfg, st), q, st.k_pool[0], st.v_pool[0], perm, pos)
    b = oracle64.attention(dims_of(cfgc, stc), q, stc.k_pool[0], stc.v_pool[0], stc.page_table[0], pos)
    assert np.array_equal(a, b)


def test_attention_brute_force_small(oracle64):
    """Brute force over every position on a tiny case, in float64 numpy."""
    pos = 6
    cfg, st, rng = _attn_setup(pos, nq=4, nkv=2, d=8, page_perm=np.array([1, 0], np.int32))
    perm = st.page_table[0]
    st.k_pool[:] = (rng.standard_normal(st.k_pool.shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    st.v_pool[:] = (rng.standard_normal(st.v_pool.shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = rng.standard_normal(32)
    out = oracle64.attention(dims_of(cfg, st), q, st.k_pool[0], st.v_pool[0], perm, pos).reshape(4, 8)
    for h in range(4):
        g = h // 2
        K = np.stack([bf16_to_f64(st.k_pool[0, perm[j // 4], g, j % 4]) for j in range(pos + 1)])
        V = np.stack([bf16_to_f64(st.v_pool[0, perm[j // 4], g, j % 4]) for j in range(pos + 1)])
        w = scipy.special.softmax(K @ q[h * 8:(h + 1) * 8] / math.sqrt(8))
        assert np.allclose(out[h], w @ V, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- whole model

def _fresh(cfg):
    return synthetic.make_model(cfg), synthetic.make_state(cfg)


def test_zero_residual_weights_reduce_to_embedding_logits(oracle64):
    """With Wo = Wdown = 0 the residual stream stays the embedding row, so the
    logits are E . rmsnorm(E[t]) and the greedy token is t itself."""
    cfg = synthetic.workload("tiny-2l")
    m, st = _fresh(cfg)
    m.weights["wo"][:] = 0
    m.weights["w_down"][:] = 0
    r = oracle64.decode_step(m, st.copy(), want_hidden=True)
    t = int(st.tokens[0])
    E = bf16_to_f64(m.weights["embed"])
    assert np.array_equal(r["hidden"][0], E[t])
    u = E[t] / math.sqrt(np.mean(E[t] ** 2) + cfg.rms_eps)
    assert np.allclose(r["logits"][0], E @ u, rtol=1e-12, atol=1e-12)
    assert r["tokens"][0] == t


def test_first_position_layer_closed_form(oracle64):
    """At position 0 RoPE is the identity and the softmax has one term, so one
    layer with Wdown = 0 is x + Wo . o with o_h = bf16(Wv u)[h / G]; the new
    cache entries are bf16(Wk u) and bf16(Wv u)."""
    cfg = small_cfg(has_embed=False, vocab=0, kv_len=0, n_layers=1)
    m, st = _fresh(cfg)
    m.weights["w_down"][:] = 0
    st0 = st.copy()
    r = oracle64.decode_step(m, st, want_hidden=True)
    H, nq, nkv, d = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    x = st0.hidden_in[0].astype(np.float64)
    u = x / math.sqrt(np.mean(x * x) + cfg.rms_eps)
    qkv = bf16_to_f64(m.weights["wqkv"][0]) @ u
    k = qkv[nq * d:(nq + nkv) * d].astype(np.float32)
    v = qkv[(nq + nkv) * d:].astype(np.float32)
    kb, vb = torch_bf16_rne(k), torch_bf16_rne(v)
    assert np.array_equal(st.k_pool[0, 0, :, 0, :].reshape(-1), kb)
    assert np.array_equal(st.v_pool[0, 0, :, 0, :].reshape(-1), vb)
    o = np.concatenate([bf16_to_f64(vb[(h // (nq // nkv)) * d:((h // (nq // nkv)) + 1) * d]) for h in range(nq)])
    ref = x + bf16_to_f64(m.weights["wo"][0]) @ o
    assert np.allclose(r["hidden"][0], ref, rtol=1e-12, atol=1e-12)


def test_mlp_block_closed_form(oracle64):
    """With Wo = 0 the attention adds nothing; the layer is then
    x + Wdown (silu(Wgate u) * (Wup u)), u = rmsnorm(x)."""
    cfg = small_cfg(has_embed=False, vocab=0, kv_len=7)
    m, st = _fresh(cfg)
    m.weights["wo"][:] = 0
    x = st.hidden_in[0].astype(np.float64)
    r = oracle64.decode_step(m, st.copy(), want_hidden=True)
    u = x / math.sqrt(np.mean(x * x) + cfg.rms_eps)
    g = bf16_to_f64(m.weights["w_gate"][0]) @ u
    up = bf16_to_f64(m.weights["w_up"][0]) @ u
    a = g * scipy.special.expit(g) * up
    ref = x + bf16_to_f64(m.weights["w_down"][0]) @ a
    assert np.allclose(r["hidden"][0], ref, rtol=1e-12, atol=1e-12)


def _complex_rope(v, pos, theta):
    """Rotate-half RoPE written as complex multiplication: element i < d/2
    pairs with i + d/2 as the complex number v_i + 1j v_(i+d/2), turned by
    the angle pos * theta^(-2i/d). v: [heads, d] float64."""
    d = v.shape[-1]
    half = d // 2
    z = v[..., :half] + 1j * v[..., half:]
    ang = pos * theta ** (-2.0 * np.arange(half) / d)
    z = z * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def _pool_rows(st, l, b, g, n, T):
    """K and V rows 0..n-1 of request b, kv head g, layer l, read through the
    page table, as float64 [n, d]."""
    pr = st.page_table[b]
    K = np.stack([bf16_to_f64(st.k_pool[l, pr[j // T], g, j % T]) for j in range(n)])
    V = np.stack([bf16_to_f64(st.v_pool[l, pr[j // T], g, j % T]) for j in range(n)])
    return K, V


def _attention_block_ref(m, st_after, l, x, p, cfg):
    """x + Wo . attention for layer l at position p, in float64, from the
    cache as it stands after the step (the new entry included): scores of
    R(p) q_h against the stored keys, softmax over positions 0..p (library
    routine), weights times the stored values."""
    H, nq, nkv, d = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = nq // nkv
    wn = bf16_to_f64(m.weights["attn_norm"][l])
    u = x / math.sqrt(np.mean(x * x) + cfg.rms_eps) * wn
    qkv = bf16_to_f64(m.weights["wqkv"][l]) @ u
    q = _complex_rope(qkv[:nq * d].reshape(nq, d), p, cfg.rope_theta)
    o = np.empty((nq, d))
    for h in range(nq):
        K, V = _pool_rows(st_after, l, 0, h // G, p + 1, cfg.page_tokens)
        o[h] = scipy.special.softmax(K @ q[h] / math.sqrt(d)) @ V
    return x + bf16_to_f64(m.weights["wo"][l]) @ o.reshape(-1), qkv


def _mlp_block_ref(m, l, x, cfg):
    wn = bf16_to_f64(m.weights["mlp_norm"][l])
    u = x / math.sqrt(np.mean(x * x) + cfg.rms_eps) * wn
    g = bf16_to_f64(m.weights["w_gate"][l]) @ u
    up = bf16_to_f64(m.weights["w_up"][l]) @ u
    return x + bf16_to_f64(m.weights["w_down"][l]) @ (g * scipy.special.expit(g) * up)


def _appended_ok(got_u16, want_f64, prec):
    """The appended bf16 entry against bf16-RNE of the float64 reference:
    exact for the double build; within one bf16 step for the single build,
    whose own rounding of the sum may land on the other side of a halfway
    point."""
    want = torch_bf16_rne(want_f64.astype(np.float32))
    if prec == "f64":
        return np.array_equal(got_u16, want)
    k = lambda a: np.where(a.astype(np.int32) & 0x8000, -(a.astype(np.int32) & 0x7fff), a.astype(np.int32))
    return int(np.max(np.abs(k(got_u16) - k(want)))) <= 1


def _randomise_norms(m, seed):
    """Distinct norm weights per layer (bf16 in [0.5, 1.5)), so that a layer
    reading another layer's norm weight gives another result."""
    rng = np.random.default_rng(seed)
    for key in ("attn_norm", "mlp_norm"):
        w = m.weights[key]
        w[:] = torch_bf16_rne(rng.uniform(0.5, 1.5, size=w.shape).astype(np.float32))


@pytest.mark.parametrize("prec", ["f64", "f32"])
def test_step_rope_at_later_position(prec, oracle64, oracle32):
    """At position p > 0 inside a full step: the appended key is
    bf16(R(p) Wk u) and the value bf16(Wv u), with R(p) written as complex
    rotations; with Wdown = 0 the layer's output is x + Wo . softmax(R(p) q .
    K^T / 8) V over the stored cache, all in float64. Rotating q or k at the
    wrong position, or storing an unrotated key, fails it."""
    ora = oracle64 if prec == "f64" else oracle32
    cfg = small_cfg(has_embed=False, vocab=0, kv_len=37, n_layers=1, head_dim=16, hidden=64,
                    page_tokens=4, cid=105, paged_random=True)
    m, st = _fresh(cfg)
    m.weights["w_down"][:] = 0
    _randomise_norms(m, 5)
    p = int(st.kv_lens[0])
    x = st.hidden_in[0].astype(np.float64)
    r = ora.decode_step(m, st, want_hidden=True)
    assert r["rc"] == 0
    ref, qkv = _attention_block_ref(m, st, 0, x, p, cfg)
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    k_new = _complex_rope(qkv[nq * d:(nq + nkv) * d].reshape(nkv, d), p, cfg.rope_theta).reshape(-1)
    v_new = qkv[(nq + nkv) * d:]
    pr = st.page_table[0]
    got_k = st.k_pool[0, pr[p // 4], :, p % 4, :].reshape(-1)
    got_v = st.v_pool[0, pr[p // 4], :, p % 4, :].reshape(-1)
    assert _appended_ok(got_k, k_new, prec)
    assert _appended_ok(got_v, v_new, prec)
    tol = 1e-12 if prec == "f64" else 2e-5
    assert np.allclose(r["hidden"][0], ref, rtol=tol, atol=tol)


@pytest.mark.parametrize("prec", ["f64", "f32"])
def test_two_layers_each_read_their_own_weights_and_cache(prec, oracle64, oracle32):
    """Two layers with distinct weights, norm weights and cache contents.
    Layer 0 keeps only its attention block's cache append (Wo = Wdown = 0),
    layer 1 only its attention block (Wdown = 0): the output is
    x + Wo1 . attention1(x) with layer 1's weights over layer 1's cache, and
    both layers' appended entries are checked. A step that reads layer 0's
    weights or pool for layer 1 fails it."""
    ora = oracle64 if prec == "f64" else oracle32
    cfg = small_cfg(has_embed=False, vocab=0, kv_len=22, n_layers=2, head_dim=16, hidden=64,
                    page_tokens=4, cid=106, paged_random=True)
    m, st = _fresh(cfg)
    m.weights["wo"][0] = 0
    m.weights["w_down"][:] = 0
    _randomise_norms(m, 6)
    p = int(st.kv_lens[0])
    x = st.hidden_in[0].astype(np.float64)
    r = ora.decode_step(m, st, want_hidden=True)
    assert r["rc"] == 0
    ref, qkv1 = _attention_block_ref(m, st, 1, x, p, cfg)
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    pr = st.page_table[0]
    for l in range(2):
        wn = bf16_to_f64(m.weights["attn_norm"][l])
        u = x / math.sqrt(np.mean(x * x) + cfg.rms_eps) * wn
        qkv = bf16_to_f64(m.weights["wqkv"][l]) @ u
        k_new = _complex_rope(qkv[nq * d:(nq + nkv) * d].reshape(nkv, d), p, cfg.rope_theta).reshape(-1)
        assert _appended_ok(st.k_pool[l, pr[p // 4], :, p % 4, :].reshape(-1), k_new, prec), l
        assert _appended_ok(st.v_pool[l, pr[p // 4], :, p % 4, :].reshape(-1), qkv[(nq + nkv) * d:], prec), l
    tol = 1e-12 if prec == "f64" else 2e-5
    assert np.allclose(r["hidden"][0], ref, rtol=tol, atol=tol)


@pytest.mark.parametrize("prec", ["f64", "f32"])
def test_two_layer_mlp_chain_closed_form(prec, oracle64, oracle32):
    """With Wo = 0 in both layers, two layers are two MLP blocks in a row,
    each with its own norm weight and matrices: x2 = m1(m0(x)), m_l(x) =
    x + Wdown_l (silu(Wgate_l u) * (Wup_l u)), u = rmsnorm(x) * w_l."""
    ora = oracle64 if prec == "f64" else oracle32
    cfg = small_cfg(has_embed=False, vocab=0, kv_len=9, n_layers=2, cid=107)
    m, st = _fresh(cfg)
    m.weights["wo"][:] = 0
    _randomise_norms(m, 7)
    x = st.hidden_in[0].astype(np.float64)
    r = ora.decode_step(m, st, want_hidden=True)
    assert r["rc"] == 0
    ref = _mlp_block_ref(m, 1, _mlp_block_ref(m, 0, x, cfg), cfg)
    tol = 1e-12 if prec == "f64" else 2e-5
    assert np.allclose(r["hidden"][0], ref, rtol=tol, atol=tol)


def test_batch_requests_are_independent(oracle64):
    cfg = small_cfg(batch=3, kv_len_range=(2, 11), paged_random=True, n_layers=2, cid=102)
    m, st = _fresh(cfg)
    full = oracle64.decode_step(m, st.copy())
    for b in range(3):
        one = synthetic.State(1, st.tokens[b:b + 1].copy(), st.kv_lens[b:b + 1].copy(),
                              st.k_pool.copy(), st.v_pool.copy(), st.page_table[b:b + 1].copy(),
                              st.n_pages, None)
        r = oracle64.decode_step(m, one)
        assert np.array_equal(r["logits"][0], full["logits"][b])
        assert r["tokens"][0] == full["tokens"][b]


def test_two_steps_match_recomputation_from_appended_cache(oracle64):
    cfg = small_cfg(n_layers=2, kv_len=9, steps=2)
    m, st = _fresh(cfg)
    s1 = oracle64.decode_step(m, st)
    st.tokens = s1["tokens"].copy()
    st.kv_lens = st.kv_lens + 1
    snapshot = st.copy()
    s2 = oracle64.decode_step(m, st)
    s2b = oracle64.decode_step(m, snapshot)
    assert np.array_equal(s2["logits"], s2b["logits"])
    # step 2 must see step 1's appended entry: clobbering it changes the result
    snap2 = st.copy()
    snap2.kv_lens = snapshot.kv_lens.copy()
    snap2.k_pool[:, 0, :, 9, :] ^= 0x0100
    s2c = oracle64.decode_step(m, snap2)
    assert not np.array_equal(s2c["logits"], s2["logits"])


def test_invalid_inputs_are_rejected(oracle64):
    cfg = small_cfg()
    m, st = _fresh(cfg)
    bad = st.copy()
    bad.kv_lens[:] = bad.page_table.shape[1] * cfg.page_tokens
    assert oracle64.decode_step(m, bad)["rc"] == -1
    bad = st.copy()
    bad.tokens[:] = cfg.vocab
    assert oracle64.decode_step(m, bad)["rc"] == -1


def test_single_precision_build_tracks_double(oracle64, oracle32):
    cfg = synthetic.workload("tiny-2l")
    m, st = _fresh(cfg)
    a = oracle64.decode_step(m, st.copy())
    b = oracle32.decode_step(m, st.copy())
    assert np.max(np.abs(a["logits"] - b["logits"])) < 1e-4
    assert a["tokens"][0] == b["tokens"][0]
