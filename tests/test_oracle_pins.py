"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test ties an oracle function to something other than itself: values the
pages print (byte counts), hand-worked cases, closed forms, exact rational
arithmetic of the page's FMA rearrangement, or brute force on tiny inputs.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            out[k] = v
    return out


# --------------------------------------------------------------------------
# Layout byte counts printed on the pages
# --------------------------------------------------------------------------

def test_layout_sizes_match_printed_values():
    rows = {}
    with open(os.path.join(GOLDEN, "layout_sizes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, val, unit, tol, *_ = line.split()
                rows[name] = (float(val), float(tol))
    e4 = oracle.expert_bytes(4096, 1024, 4)
    e2 = oracle.expert_bytes(4096, 1024, 2)
    assert e4 == 7_077_888 and e2 == 3_932_160
    got = {
        "expert_4bit_MiB": e4 / 2 ** 20,
        "io_per_token_2bit_MB": 60 * 4 * e2 / 1e6,
        "total_2bit_GB": 60 * 512 * e2 / 1e9,
    }
    for k, (val, tol) in rows.items():
        assert abs(got[k] - val) <= tol * val, (k, got[k], val)


def test_layout_offsets_are_ordered_and_aligned():
    off = oracle.expert_offsets(4096, 1024, 4)
    names = ["gate_codes", "up_codes", "down_codes", "gate_sb", "up_sb", "down_sb"]
    pos = 0
    for n in names:
        o, s = off[n]
        assert o == pos and o % 256 == 0
        pos += s
    assert off["total"] == pos
    # other group multiples
    assert oracle.expert_bytes(128, 64, 2) == 2 * 64 * 128 // 4 + 128 * 64 // 4 + 4 * (2 * 64 * 2 + 128)


# --------------------------------------------------------------------------
# Dequantisation: hand-built cases
# --------------------------------------------------------------------------

def _hexrow(words):
    return np.frombuffer(bytes.fromhex("".join(words)), dtype=np.uint8)


def test_dequant_handmade_4bit():
    g = _golden_kv("dequant_handmade.txt")
    cols = int(g["A.cols"][0])
    codes = np.stack([_hexrow(g["A.row0"]), _hexrow(g["A.row1"])])
    sb = np.array([[int(g["A.sb0"][0], 16)], [int(g["A.sb1"][0], 16)]], dtype=np.uint32)
    W = oracle.dequant(codes, sb, cols, 4)
    np.testing.assert_array_equal(W[0, :16], [float(v) for v in g["A.W0_first16"]])
    np.testing.assert_array_equal(W[1, :4], [float(v) for v in g["A.W1_first4"]])
    y = oracle.qgemv(codes, sb, np.ones(cols), 4)
    np.testing.assert_array_equal(y, [float(v) for v in g["A.y_ones"]])


def test_dequant_handmade_2bit_two_groups():
    g = _golden_kv("dequant_handmade.txt")
    cols = int(g["B.cols"][0])
    codes = _hexrow(g["B.row0"])[None, :]
    sb = np.array([[int(v, 16) for v in g["B.sb0"]]], dtype=np.uint32)
    W = oracle.dequant(codes, sb, cols, 2)
    np.testing.assert_array_equal(W[0, :4], [float(v) for v in g["B.W0_first4"]])
    np.testing.assert_array_equal(W[0, 64:68], [float(v) for v in g["B.W0_64_to_67"]])
    np.testing.assert_array_equal(oracle.qgemv(codes, sb, np.ones(cols), 2), [float(g["B.y_ones"][0])])


@pytest.mark.parametrize("bits", [2, 4])
def test_unit_vector_picks_one_column(bits):
    """x = e_k returns column k of W: catches bit-order and transposition mistakes."""
    rng = np.random.default_rng(7)
    rows, cols = 5, 128
    codes = rng.integers(0, 256, size=(rows, cols * bits // 8), dtype=np.uint8)
    sb = np.zeros((rows, cols // 64), dtype=np.uint32) | np.uint32(0x3F80)  # scale 1, bias 0
    for k in (0, 1, 2, 3, 5, 63, 64, 127):
        x = np.zeros(cols)
        x[k] = 1.0
        y = oracle.qgemv(codes, sb, x, bits)
        byte = codes[:, (k * bits) // 8].astype(np.int64)
        expect = (byte >> ((k * bits) % 8)) & ((1 << bits) - 1)
        np.testing.assert_array_equal(y, expect.astype(np.float64))


@pytest.mark.parametrize("bits", [2, 4])
def test_unit_scale_zero_bias_is_integer_matmul(bits):
    """scale 1, bias 0: the GEMV is an integer matrix times an integer vector, exact."""
    rng = np.random.default_rng(11)
    rows, cols = 9, 192
    q = rng.integers(0, 1 << bits, size=(rows, cols))
    packed = np.zeros((rows, cols * bits // 8), dtype=np.uint8)
    per = 8 // bits
    for k in range(cols):  # pack by hand with the documented rule
        packed[:, k // per] |= (q[:, k] << ((k % per) * bits)).astype(np.uint8)
    sb = np.full((rows, cols // 64), 0x3F80, dtype=np.uint32)
    x = rng.integers(-1000, 1000, size=cols)
    y = oracle.qgemv(packed, sb, x.astype(np.float64), bits)
    np.testing.assert_array_equal(y, (q @ x).astype(np.float64))


@pytest.mark.parametrize("bits", [2, 4])
def test_constant_codes_closed_form(bits):
    """All codes c, constant scale s and bias b: y_n = (c*s + b) * sum(x)."""
    rows, cols = 3, 256
    c = (1 << bits) - 2
    byte = 0
    for j in range(8 // bits):
        byte |= c << (j * bits)
    codes = np.full((rows, cols * bits // 8), byte, dtype=np.uint8)
    s_bits, b_bits = 0x3E00, 0xBD00          # 0.125 and -0.03125
    sb = np.full((rows, cols // 64), s_bits | (b_bits << 16), dtype=np.uint32)
    x = np.random.default_rng(3).standard_normal(cols)
    y = oracle.qgemv(codes, sb, x, bits)
    np.testing.assert_allclose(y, (c * 0.125 - 0.03125) * x.sum() * np.ones(rows), rtol=1e-13)


# --------------------------------------------------------------------------
# The FMA rearrangement of the page is an identity (exact rational arithmetic)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 4])
def test_fma_rearrangement_identity_exact(bits):
    """Sum over k of (q*s + b)*x  ==  sum of fma(q, s*x, b*x)  ==  per-group
    s*sum(q*x) + b*sum(x), exactly in rationals; the oracle's float64 value
    agrees to rounding.  Source: "flash-moe 소개", section
    "FMA 최적화 역양자화 커널" (the (nibble*scale+bias)*x -> fma(nibble, scale*x,
    bias*x) rearrangement)."""
    rng = np.random.default_rng(5 + bits)
    rows, cols = 2, 128
    codes = rng.integers(0, 256, size=(rows, cols * bits // 8), dtype=np.uint8)
    s16 = rng.integers(0x3A00, 0x3D00, size=(rows, cols // 64)).astype(np.uint32)
    b16 = rng.integers(0xBC00, 0xBD00, size=(rows, cols // 64)).astype(np.uint32)
    sb = s16 | (b16 << 16)
    x = rng.standard_normal(cols)

    def bf(u):
        return Fraction(float(np.array([u << 16], dtype=np.uint32).view(np.float32)[0]))

    per = 8 // bits
    for n in range(rows):
        q = [(int(codes[n, k // per]) >> ((k % per) * bits)) & ((1 << bits) - 1) for k in range(cols)]
        xs = [Fraction(float(v)) for v in x]
        s = [bf(int(s16[n, g])) for g in range(cols // 64)]
        b = [bf(int(b16[n, g])) for g in range(cols // 64)]
        naive = sum((q[k] * s[k // 64] + b[k // 64]) * xs[k] for k in range(cols))
        fma_form = sum(q[k] * (s[k // 64] * xs[k]) + (b[k // 64] * xs[k]) for k in range(cols))
        grouped = sum(s[g] * sum(q[k] * xs[k] for k in range(64 * g, 64 * g + 64))
                      + b[g] * sum(xs[64 * g:64 * g + 64]) for g in range(cols // 64))
        assert naive == fma_form == grouped
        y = oracle.qgemv(codes[n:n + 1], sb[n:n + 1], x, bits)[0]
        assert abs(y - float(naive)) <= 1e-13 * max(1.0, abs(float(naive)))


# --------------------------------------------------------------------------
# Router, softmax and top-K
# --------------------------------------------------------------------------

def _bf16(v):
    return (np.array(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_router_handmade_with_ties():
    # E=6, H=2, x=(1,1): logits [0.5, 1, 2, -1, 0.5, 1] (all exact in bf16)
    Wr = _bf16([[0.5, 0.0], [1.0, 0.0], [0.0, 2.0], [-1.0, 0.0], [0.25, 0.25], [0.5, 0.5]])
    logits = oracle.router_logits(Wr, np.array([1.0, 1.0]))
    np.testing.assert_array_equal(logits, [0.5, 1, 2, -1, 0.5, 1])
    idx, w = oracle.router_topk(logits, 4)
    assert list(idx) == [2, 1, 5, 0]          # ties go to the lower index
    idx2, w2 = oracle.router_topk(logits, 2)
    assert list(idx2) == [2, 1]
    e = math.e
    np.testing.assert_allclose(w2, [e / (1 + e), 1 / (1 + e)], rtol=1e-15)


def _brute_force_topk_set(logits, k):
    p = np.exp(logits - logits.max())
    p /= p.sum()
    best, best_mass = None, -1.0
    for subset in itertools.combinations(range(logits.size), k):
        mass = float(sum(p[list(subset)]))
        if mass > best_mass:
            best, best_mass = subset, mass
    return set(best), p


@pytest.mark.parametrize("E,k", [(4, 1), (6, 2), (8, 4), (10, 3), (10, 10)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 31 + k)
    for _ in range(20):
        logits = rng.standard_normal(E) * 3
        idx, w = oracle.router_topk(logits, k)
        best, p = _brute_force_topk_set(logits, k)
        assert set(idx.tolist()) == best
        assert all(logits[idx[i]] >= logits[idx[i + 1]] for i in range(k - 1))
        assert abs(w.sum() - 1.0) < 1e-15
        np.testing.assert_allclose(w, p[idx] / p[idx].sum(), rtol=1e-13)
        # invariance to a shift of every logit
        idx_s, w_s = oracle.router_topk(logits + 123.0, k)
        assert list(idx_s) == list(idx)
        np.testing.assert_allclose(w_s, w, rtol=1e-12)


def test_topk_decides_in_float32():
    # two logits that differ in float64 but round to the same float32: a tie,
    # broken towards the lower index, as the fp32 kernel does
    a = 1.0
    b = 1.0 + 2.0 ** -30
    assert np.float32(a) == np.float32(b)
    idx, _ = oracle.router_topk(np.array([0.0, a, b, -1.0]), 1)
    assert list(idx) == [1]
    idx64, _ = oracle.router_topk(np.array([0.0, a, b, -1.0]), 1, decide_in=None)
    assert list(idx64) == [2]


# --------------------------------------------------------------------------
# SwiGLU, sigmoid, expert FFN, combine
# --------------------------------------------------------------------------

def test_silu_sigmoid_special_values():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15
    np.testing.assert_allclose(oracle.silu(1.0), 1.0 / (1.0 + math.exp(-1.0)), rtol=1e-15)
    # silu(z) - silu(-z) = z
    z = np.linspace(-5, 5, 11)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, atol=1e-14)


def _const_expert_block(H, I, bits, gate, up, down):
    """Expert whose three matrices are constant: (code, scale_bits, bias_bits)."""
    blk = np.zeros(oracle.expert_bytes(H, I, bits), dtype=np.uint8)
    off = oracle.expert_offsets(H, I, bits)
    for name, (c, s, b) in (("gate", gate), ("up", up), ("down", down)):
        o, n = off[name + "_codes"]
        byte = 0
        for j in range(8 // bits):
            byte |= c << (j * bits)
        blk[o:o + n] = byte
        o, n = off[name + "_sb"]
        blk[o:o + n] = np.full(n // 4, s | (b << 16), dtype=np.uint32).view(np.uint8)
    return blk


@pytest.mark.parametrize("bits", [2, 4])
def test_expert_ffn_closed_form(bits):
    """Constant matrices: gate W=1, up W=2, down W=0.5 and sum(x)=1 give
    a = 1, u = 2, h = silu(1)*2, y_n = I * 0.5 * h = I*silu(1).  A swap of
    gate and up (silu on the up projection) would give I*silu(2)/2 instead."""
    H, I = 128, 64
    gate = (2, 0x3F00, 0x0000)      # 2*0.5 + 0 = 1
    up = (1, 0x3F80, 0x3F80)        # 1*1 + 1 = 2
    down = (3, 0x3E80, 0xBE80)      # 3*0.25 - 0.25 = 0.5
    blk = _const_expert_block(H, I, bits, gate, up, down)
    x = np.full(H, 1.0 / H)
    y, mid = oracle.expert_ffn(blk, x, H, I, bits, return_intermediates=True)
    np.testing.assert_allclose(mid["a"], 1.0, rtol=1e-14)
    np.testing.assert_allclose(mid["u"], 2.0, rtol=1e-14)
    np.testing.assert_allclose(y, I * oracle.silu(1.0), rtol=1e-13)
    assert abs(I * oracle.silu(2.0) / 2 - I * oracle.silu(1.0)) > 1.0


def test_combine_special_cases():
    H, K = 8, 3
    rng = np.random.default_rng(2)
    ys = rng.standard_normal((K, H))
    y_sh = rng.standard_normal(H)
    x = rng.standard_normal(H)
    r = rng.standard_normal(H)
    g0 = np.zeros(H, dtype=np.uint16)                # g = 0 -> gamma = 1/2
    out = oracle.combine_residual_gate(ys, np.zeros(K), y_sh, g0, x, r)
    np.testing.assert_allclose(out, r + 0.5 * y_sh, rtol=1e-15)
    out1 = oracle.combine_residual_gate(ys[:1], np.ones(1), np.zeros(H), g0, x, r)
    np.testing.assert_allclose(out1, r + ys[0], rtol=1e-15)
    # a large gate saturates the sigmoid: gamma -> 1 ; negative -> 0
    big = _bf16(np.full(H, 64.0))
    xs = np.ones(H)
    np.testing.assert_allclose(oracle.combine_residual_gate(ys, np.zeros(K), y_sh, big, xs, r),
                               r + y_sh, rtol=1e-12)
    np.testing.assert_allclose(oracle.combine_residual_gate(ys, np.zeros(K), y_sh, big, -xs, r),
                               r, rtol=1e-12, atol=1e-12)
    w = np.array([0.5, 0.25, 0.25])
    out2 = oracle.combine_residual_gate(ys, w, y_sh, g0, x, r)
    np.testing.assert_allclose(out2, r + 0.5 * ys[0] + 0.25 * ys[1] + 0.25 * ys[2] + 0.5 * y_sh,
                               rtol=1e-14)


def test_rmsnorm_closed_forms():
    H = 16
    w = np.linspace(0.9, 1.1, H)
    for c in (1.0, -3.0, 1e-4):
        out = oracle.rmsnorm(np.full(H, c), w, 1e-6)
        np.testing.assert_allclose(out, c / math.sqrt(c * c + 1e-6) * w, rtol=1e-14)
    v = np.random.default_rng(4).standard_normal(H)
    # eps = 0: scale invariance and unit RMS with w = 1
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * v, w, 0.0), oracle.rmsnorm(v, w, 0.0), rtol=1e-14)
    o = oracle.rmsnorm(v, np.ones(H), 0.0)
    assert abs(math.sqrt(np.mean(o * o)) - 1.0) < 1e-14


# --------------------------------------------------------------------------
# Layer-level structure
# --------------------------------------------------------------------------

def _small_layer(bits, E=6, H=128, I=64, seed=1):
    rng = np.random.default_rng(seed)
    nb = oracle.expert_bytes(H, I, bits)
    off = oracle.expert_offsets(H, I, bits)
    blocks = []
    for _ in range(E + 1):
        blk = rng.integers(0, 256, size=nb, dtype=np.uint8)
        for name in ("gate_sb", "up_sb", "down_sb"):
            o, n = off[name]
            s = rng.integers(0x3A00, 0x3C80, size=n // 4).astype(np.uint32)
            b = rng.integers(0xBC00, 0xBD00, size=n // 4).astype(np.uint32)
            blk[o:o + n] = (s | (b << 16)).view(np.uint8)
        blocks.append(blk)
    router = _bf16(rng.standard_normal((E, H)) * 0.1)
    gate = _bf16(rng.standard_normal(H) * 0.1)
    return blocks[:E], blocks[E], router, gate


def test_moe_layer_zero_experts_is_residual():
    """Experts whose weights are all zero contribute nothing: out = residual."""
    H, I, bits = 128, 64, 4
    zero = np.zeros(oracle.expert_bytes(H, I, bits), dtype=np.uint8)
    router = _bf16(np.random.default_rng(0).standard_normal((5, H)))
    x = np.random.default_rng(1).standard_normal(H)
    r = np.random.default_rng(2).standard_normal(H)
    out = oracle.moe_layer(lambda e: zero, zero, router, np.zeros(H, np.uint16), x, r, H, I, bits, 2)
    np.testing.assert_array_equal(out, r)


@pytest.mark.parametrize("bits", [2, 4])
def test_moe_layer_matches_its_parts(bits):
    """The layer uses the selected experts with their renormalised weights and
    gates only the shared expert (checked against the parts computed one by one)."""
    H, I, K = 128, 64, 2
    experts, shared, router, gate = _small_layer(bits)
    x = np.random.default_rng(9).standard_normal(H)
    out, d = oracle.moe_layer(lambda e: experts[e], shared, router, gate, x, x, H, I, bits, K,
                              return_details=True)
    logits = oracle.bf16_bits_to_f64(router) @ x
    order = np.argsort(-logits, kind="stable")[:K]
    assert list(d["idx"]) == list(order)
    p = np.exp(logits - logits.max())
    w = p[order] / p[order].sum()
    gamma = 1 / (1 + np.exp(-(oracle.bf16_bits_to_f64(gate) @ x)))
    expect = x + sum(w[i] * oracle.expert_ffn(experts[order[i]], x, H, I, bits) for i in range(K)) \
        + gamma * oracle.expert_ffn(shared, x, H, I, bits)
    np.testing.assert_allclose(out, expect, rtol=1e-12)


def test_batched_rows_equal_single_token():
    H, I, bits, K = 128, 64, 4, 2
    experts, shared, router, gate = _small_layer(bits, seed=3)
    X = np.random.default_rng(5).standard_normal((3, H))
    out = oracle.moe_layer_batched(lambda e: experts[e], shared, router, gate, X, X, H, I, bits, K)
    for t in range(3):
        np.testing.assert_array_equal(
            out[t], oracle.moe_layer(lambda e: experts[e], shared, router, gate, X[t], X[t],
                                     H, I, bits, K))


def test_stack_of_zero_layers_keeps_h():
    H, I, bits = 128, 64, 2
    zero = np.zeros(oracle.expert_bytes(H, I, bits), dtype=np.uint8)
    router = _bf16(np.random.default_rng(0).standard_normal((4, H)))
    layers = [dict(get_expert=lambda e: zero, shared_block=zero, router=router,
                   shared_gate=np.zeros(H, np.uint16), norm_w=np.ones(H)) for _ in range(3)]
    h0 = np.random.default_rng(8).standard_normal(H)
    np.testing.assert_array_equal(oracle.moe_stack(layers, h0, H, I, bits, 2), h0)


def test_stack_feeds_normalised_input():
    """One layer with constant experts: x = rmsnorm(h0) enters the experts,
    h0 (not x) is the residual."""
    H, I, bits = 128, 64, 4
    blk = _const_expert_block(H, I, bits, (2, 0x3F00, 0), (1, 0x3F80, 0x3F80), (3, 0x3E80, 0xBE80))
    router = _bf16(np.zeros((2, H)))
    h0 = np.full(H, 3.0)
    w = np.full(H, 1.0 / H)   # x = rmsnorm(h0) * w = (3/sqrt(9+eps)) / H per entry, sum(x) ~ 1
    layer = dict(get_expert=lambda e: blk, shared_block=blk, router=router,
                 shared_gate=np.zeros(H, np.uint16), norm_w=w)
    out = oracle.moe_stack([layer], h0, H, I, bits, 1)
    S = 3.0 / math.sqrt(9.0 + 1e-6)        # sum of x
    y = I * 0.5 * 2.0 * S * oracle.silu(S)  # constant-expert output for sum(x) = S
    np.testing.assert_allclose(out, h0 + y + 0.5 * y, rtol=1e-12)


# --------------------------------------------------------------------------
# GatedDeltaNet recurrence
# --------------------------------------------------------------------------

def _gdn_inputs(rng, heads, dk, dv):
    S = rng.standard_normal((heads, dk, dv))
    q = rng.standard_normal((heads, dk))
    k = rng.standard_normal((heads, dk))
    v = rng.standard_normal((heads, dv))
    return S, q, k, v


def test_gdn_delta_rule_stores_the_value_at_its_key():
    """beta = 1 and a unit key: afterwards the key recalls exactly v, whatever the
    decay and the (non-symmetric) state held before -- the defining property of
    the delta rule.  A transposed state, a decay missing from the recall or a
    wrong sign all break it."""
    rng = np.random.default_rng(11)
    S, q, k, v = _gdn_inputs(rng, 3, 5, 4)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    alpha = np.array([1.0, 0.5, 0.9])
    S2, _ = oracle.gdn_step(S, q, k, v, alpha, np.ones(3))
    for h in range(3):
        recall = np.array([sum(S2[h, i, j] * k[h, i] for i in range(5)) for j in range(4)])
        np.testing.assert_allclose(recall, v[h], rtol=0, atol=1e-12)


def test_gdn_zero_state_closed_form():
    """From a zero state: S' = beta k v^T and o = beta (k . q) v."""
    rng = np.random.default_rng(12)
    _, q, k, v = _gdn_inputs(rng, 2, 4, 3)
    beta = np.array([0.25, 0.75])
    S2, o = oracle.gdn_step(np.zeros((2, 4, 3)), q, k, v, np.array([0.3, 0.6]), beta)
    for h in range(2):
        for i in range(4):
            for j in range(3):
                assert S2[h, i, j] == pytest.approx(beta[h] * k[h, i] * v[h, j], rel=1e-14)
        kq = sum(k[h, i] * q[h, i] for i in range(4))
        np.testing.assert_allclose(o[h], beta[h] * kq * v[h], rtol=1e-13)


def test_gdn_gates_off_and_decay_only():
    """beta = 0: the state only decays (alpha = 1: it is unchanged) and the
    output is the decayed state read at q, summed by hand."""
    rng = np.random.default_rng(13)
    S, q, k, v = _gdn_inputs(rng, 2, 3, 4)
    for alpha in (1.0, 0.25):
        S2, o = oracle.gdn_step(S, q, k, v, np.full(2, alpha), np.zeros(2))
        np.testing.assert_array_equal(S2, alpha * S)
        for h in range(2):
            for j in range(4):
                assert o[h, j] == pytest.approx(alpha * sum(S[h, i, j] * q[h, i] for i in range(3)), rel=1e-13)


def test_gdn_orthogonal_keys_do_not_interfere():
    """A state holding values at orthonormal keys (S = sum_m k_m v_m^T): writing a
    new value at key 0 leaves what the other keys recall untouched, and the output
    for q = key m is the value stored there."""
    rng = np.random.default_rng(14)
    dk, dv = 6, 5
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q.T                                   # rows: orthonormal keys
    vals = rng.standard_normal((dk, dv))
    S = sum(np.outer(keys[m], vals[m]) for m in range(dk))[None]
    vnew = rng.standard_normal((1, dv))
    for m in range(1, dk):
        S2, o = oracle.gdn_step(S, keys[m][None], keys[0][None], vnew, np.ones(1), np.ones(1))
        np.testing.assert_allclose(o[0], vals[m], atol=1e-12)
    np.testing.assert_allclose(S2[0].T @ keys[0], vnew[0], atol=1e-12)


def test_gdn_steps_compose():
    """Two tokens through the recurrence equal the explicit two-step formula
    S2 = a2 (a1 S + k1 d1^T) + k2 d2^T with d_t = b_t (v_t - recall), written out
    element by element on a tiny case."""
    rng = np.random.default_rng(15)
    dk, dv = 3, 2
    S = rng.standard_normal((1, dk, dv))
    qs, ks, vs = rng.standard_normal((2, dk)), rng.standard_normal((2, dk)), rng.standard_normal((2, dv))
    a, b = [0.7, 0.9], [0.4, 0.8]
    St = S.copy()
    for t in range(2):
        St, _ = oracle.gdn_step(St, qs[t][None], ks[t][None], vs[t][None], np.array([a[t]]), np.array([b[t]]))
    M = [[S[0, i, j] for j in range(dv)] for i in range(dk)]
    for t in range(2):
        M = [[a[t] * M[i][j] for j in range(dv)] for i in range(dk)]
        rec = [sum(M[i][j] * ks[t][i] for i in range(dk)) for j in range(dv)]
        d = [b[t] * (vs[t][j] - rec[j]) for j in range(dv)]
        M = [[M[i][j] + ks[t][i] * d[j] for j in range(dv)] for i in range(dk)]
    np.testing.assert_allclose(St[0], np.array(M), rtol=1e-13)


# --------------------------------------------------------------------------
# RoPE and full-attention decode
# --------------------------------------------------------------------------

def test_rope_hand_case_and_pass_through():
    """D = 4, rot_dim = 2: the pair (x0, x1) turns by pos radians (theta^0 = 1),
    x2 and x3 pass through; pos = 0 is the identity."""
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    r = oracle.rope(x, 3, 10000.0, 2)
    c, s = math.cos(3.0), math.sin(3.0)
    np.testing.assert_allclose(r[0], [c - 2 * s, 2 * c + s, 3.0, 4.0], rtol=1e-15)
    np.testing.assert_array_equal(oracle.rope(x, 0, 10000.0, 4), x)


def test_rope_second_frequency_by_hand():
    """rot_dim = 4, theta = 100: pair 1 is (x1, x3) and turns by pos * 100^(-1/2)."""
    x = np.array([[0.0, 1.0, 0.0, 0.0]])
    r = oracle.rope(x, 5, 100.0, 4)
    a = 5 * 0.1
    np.testing.assert_allclose(r[0], [0.0, math.cos(a), 0.0, math.sin(a)], atol=1e-15)


def test_rope_is_relative():
    """Rotations preserve length, and rope(q, m) . rope(k, n) depends on m - n only."""
    rng = np.random.default_rng(21)
    q, k = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    for m, n in ((7, 3), (40, 36), (4, 0)):
        d1 = float(oracle.rope(q, m, 500.0, 16)[0] @ oracle.rope(k, n, 500.0, 16)[0])
        d0 = float(oracle.rope(q, m - n, 500.0, 16)[0] @ k[0])
        assert d1 == pytest.approx(d0, rel=1e-12)
        assert np.linalg.norm(oracle.rope(q, m, 500.0, 12)) == pytest.approx(np.linalg.norm(q), rel=1e-14)


def test_attn_single_key_returns_its_value():
    """At pos = 0 the only key is the token's own: o = v for every query head."""
    rng = np.random.default_rng(22)
    q, k, v = rng.standard_normal((4, 8)), rng.standard_normal((2, 8)), rng.standard_normal((2, 8))
    o, K, V = oracle.attn_decode(q, k, v, np.zeros((2, 5, 8)), np.zeros((2, 5, 8)), 0, 1e4, 8)
    for h in range(4):
        np.testing.assert_allclose(o[h], v[h // 2], rtol=1e-15)
    np.testing.assert_array_equal(V[:, 0], v)
    np.testing.assert_allclose(K[:, 0], k, rtol=1e-15)   # rotation at position 0 is the identity


def test_attn_equal_keys_average_the_values():
    """Keys identical to the token's rotated key: uniform weights, o = mean of V[0..pos]."""
    rng = np.random.default_rng(23)
    D, pos = 8, 4
    q, k, v = rng.standard_normal((2, D)), rng.standard_normal((1, D)), rng.standard_normal((1, D))
    kr = oracle.rope(k, pos, 1e4, D)
    K = np.repeat(kr[:, None, :], 6, axis=1)
    V = rng.standard_normal((1, 6, D))
    o, _, V2 = oracle.attn_decode(q, k, v, K, V, pos, 1e4, D)
    np.testing.assert_allclose(o[0], V2[0, :pos + 1].mean(axis=0), rtol=1e-12)
    np.testing.assert_allclose(o[1], o[0], rtol=1e-12)


def test_attn_brute_force_with_explicit_softmax():
    """A tiny case summed by hand with math.exp (grouping 3:1, partial rotation)."""
    rng = np.random.default_rng(24)
    Hq, Hkv, D, T, pos = 3, 1, 4, 5, 3
    q, k, v = rng.standard_normal((Hq, D)), rng.standard_normal((Hkv, D)), rng.standard_normal((Hkv, D))
    K, V = rng.standard_normal((Hkv, T, D)), rng.standard_normal((Hkv, T, D))
    o, K2, V2 = oracle.attn_decode(q, k, v, K, V, pos, 50.0, 2)
    c, s = math.cos(pos), math.sin(pos)
    def rot(x):
        return [x[0] * c - x[1] * s, x[1] * c + x[0] * s, x[2], x[3]]
    keys = [list(K[0, t]) for t in range(pos)] + [rot(k[0])]
    vals = [list(V[0, t]) for t in range(pos)] + [list(v[0])]
    for h in range(Hq):
        qh = rot(q[h])
        sc = [sum(a * b for a, b in zip(qh, key)) / 2.0 for key in keys]
        w = [math.exp(x - max(sc)) for x in sc]
        ref = [sum(w[t] * vals[t][d] for t in range(pos + 1)) / sum(w) for d in range(D)]
        np.testing.assert_allclose(o[h], ref, rtol=1e-12)
    np.testing.assert_array_equal(K2[0, pos + 1:], K[0, pos + 1:])   # rows past pos untouched


# --------------------------------------------------------------------------
# The comparison helpers every parity test relies on: rel_l2 (the bar), the
# fp32 near-tie tolerance of the top-K, and the forced-selection branch of
# moe_layer (the reference taken when a near-tie is exempted)
# --------------------------------------------------------------------------

def test_rel_l2_hand_cases():
    # ||(9,12) - (6,8)|| = ||(3,4)|| = 5 against ||(6,8)|| = 10
    assert oracle.rel_l2([9.0, 12.0], [6.0, 8.0]) == 0.5
    # the second argument is the reference: ||(3,4)|| / ||(9,12)|| = 1/3
    assert abs(oracle.rel_l2([6.0, 8.0], [9.0, 12.0]) - 1.0 / 3.0) < 1e-16
    # twice the reference is one reference-norm away
    b = np.array([1.0, -2.0, 2.0])
    assert oracle.rel_l2(2 * b, b) == 1.0
    assert oracle.rel_l2(b, b) == 0.0
    # zero reference: the absolute norm of a (||(3,4,0)|| = 5)
    assert oracle.rel_l2([3.0, 4.0, 0.0], [0.0, 0.0, 0.0]) == 5.0
    # a small error stays linear in its size: 1e-4 relative, not 1e-8
    c = np.array([0.0, 0.0, 2.0])
    assert abs(oracle.rel_l2(c + [0.0, 2e-4, 0.0], c) - 1e-4) < 1e-18
    # shapes are flattened
    assert oracle.rel_l2(np.array([[9.0], [12.0]]), np.array([6.0, 8.0])) == 0.5


def test_topk_tolerance_closed_form():
    """A 3-expert router of exact bf16 values over H = 4 inputs:
    sum_h |W[e,h] x[h]| = 4, 5 and 0, sqrt(H) = 2, so tau = 4 * 2^-24 * 2 * (4, 5, 0)."""
    Wr = _bf16([[1.0, -2.0, 0.5, 0.0], [-1.0, 1.0, 1.0, 0.25], [0.0, 0.0, 0.0, 0.0]])
    x = np.array([1.0, 1.0, -2.0, 4.0])
    tau = oracle.topk_tolerance(Wr, x)
    np.testing.assert_array_equal(tau, [2.0 ** -19, 1.25 * 2.0 ** -19, 0.0])
    # an explicit term count replaces H in the square root
    np.testing.assert_array_equal(oracle.topk_tolerance(Wr, x, n_terms=16), 2 * tau)


def test_topk_tolerance_bounds_real_fp32_error_and_is_tight():
    """On config-sized random routers, tau covers the error of sequentially
    accumulated fp32 dot products (the worst summation order a kernel could
    take) yet stays within a small factor of the largest error seen."""
    rng = np.random.default_rng(17)
    H, E = 4096, 64
    Wr = _bf16(rng.standard_normal((E, H)) * 0.02)
    W32 = oracle.bf16_bits_to_f64(Wr).astype(np.float32)
    x = rng.standard_normal(H).astype(np.float32)
    exact = oracle.router_logits(Wr, x.astype(np.float64))
    tau = oracle.topk_tolerance(Wr, x)
    seq = np.zeros(E, np.float32)
    for h in range(H):                       # one fp32 rounding per term, in order
        seq = (seq + W32[:, h] * x[h]).astype(np.float32)
    err = np.abs(seq.astype(np.float64) - exact)
    assert np.all(err <= tau)
    # generous (about 130x the largest error here) but not loose: within 500x
    assert err.max() > tau.max() / 500


def _const_layer_block(H, I, bits, down_bias_bits):
    """All codes zero; gate bias 1, up bias 1/64, down bias given, scales 1.
    With x = e_0: a = 1, u = 1/64, h = silu(1)/64, y = down_bias * I * silu(1)/64."""
    return _const_expert_block(H, I, bits, (0, 0x3F80, 0x3F80), (0, 0x3F80, 0x3C80),
                               (0, 0x3F80, down_bias_bits))


def test_moe_layer_forced_selection_by_hand():
    """force_idx picks the experts and their weights are the softmax of the
    forced logits: a forced set that is not the top-K, with experts whose
    outputs are distinct constants, checked against hand-computed values."""
    H, I, bits, K = 64, 64, 4, 2
    down = [0x3F00, 0x3F80, 0x3FC0, 0x4000, 0x4020, 0x4040]   # 0.5, 1, 1.5, 2, 2.5, 3
    blocks = [_const_layer_block(H, I, bits, d) for d in down]
    shared = _const_layer_block(H, I, bits, 0x4080)           # 4
    logit = [0.5, -1.0, 2.0, 0.25, 1.5, -0.5]
    Wr = np.zeros((6, H), np.float32)
    Wr[:, 0] = logit
    Wr = _bf16(Wr)
    gate = np.zeros(H, np.uint16)                             # gamma = 1/2
    x = np.zeros(H)
    x[0] = 1.0
    r = np.linspace(-1.0, 1.0, H)
    s1 = 1.0 / (1.0 + math.exp(-1.0))                        # silu(1)
    y = [d * I * s1 / 64 for d in (0.5, 1.0, 1.5, 2.0, 2.5, 3.0)]
    y_sh = 4.0 * I * s1 / 64

    # natural selection: experts 2 and 4 (logits 2 and 1.5)
    out_nat, d = oracle.moe_layer(lambda e: blocks[e], shared, Wr, gate, x, r, H, I, bits, K,
                                  return_details=True)
    assert list(d["idx"]) == [2, 4]
    w_nat = [1.0 / (1.0 + math.exp(-0.5)), 1.0 / (1.0 + math.exp(0.5))]
    np.testing.assert_allclose(d["w"], w_nat, rtol=1e-15)
    np.testing.assert_allclose(out_nat, r + w_nat[0] * y[2] + w_nat[1] * y[4] + 0.5 * y_sh,
                               rtol=1e-13, atol=1e-15)
    # forcing the natural set changes nothing
    out_same = oracle.moe_layer(lambda e: blocks[e], shared, Wr, gate, x, r, H, I, bits, K,
                                force_idx=[2, 4])
    np.testing.assert_array_equal(out_same, out_nat)

    # forced {0, 3}: weights softmax(0.5, 0.25), not uniform and not the full softmax
    out_f, d = oracle.moe_layer(lambda e: blocks[e], shared, Wr, gate, x, r, H, I, bits, K,
                                force_idx=[0, 3], return_details=True)
    e0, e3 = math.exp(0.5), math.exp(0.25)
    w_f = [e0 / (e0 + e3), e3 / (e0 + e3)]
    assert list(d["idx"]) == [0, 3]
    np.testing.assert_allclose(d["w"], w_f, rtol=1e-15)
    np.testing.assert_allclose(out_f, r + w_f[0] * y[0] + w_f[1] * y[3] + 0.5 * y_sh,
                               rtol=1e-13, atol=1e-15)
    # the forced order is kept: [3, 0] gives the same output with swapped weights
    _, d = oracle.moe_layer(lambda e: blocks[e], shared, Wr, gate, x, r, H, I, bits, K,
                            force_idx=[3, 0], return_details=True)
    np.testing.assert_allclose(d["w"], w_f[::-1], rtol=1e-15)


# --------------------------------------------------------------------------
# The attention step's input side: Q de-interleave and the per-head RMS norm
# --------------------------------------------------------------------------

def test_deinterleave_q_hand_case():
    qg = np.array([[1.0, 2.0, 3.0, 4.0], [5.0, 6.0, 7.0, 8.0]])
    q, gate = oracle.deinterleave_q(qg, 2)
    np.testing.assert_array_equal(q, [[1.0, 2.0], [5.0, 6.0]])
    np.testing.assert_array_equal(gate, [[3.0, 4.0], [7.0, 8.0]])
    with pytest.raises(ValueError):
        oracle.deinterleave_q(qg, 3)


def test_head_rmsnorm_hand_cases():
    # row (3, 4): mean square 12.5; row (-2, -2, -2, -2) is constant
    x = np.array([[3.0, 4.0]])
    np.testing.assert_allclose(oracle.head_rmsnorm(x, [1.0, 2.0], 0.0),
                               [[3.0 / math.sqrt(12.5), 8.0 / math.sqrt(12.5)]], rtol=1e-15)
    c = np.full((1, 4), -2.0)
    np.testing.assert_allclose(oracle.head_rmsnorm(c, np.ones(4), 1e-6), -2.0 / math.sqrt(4.0 + 1e-6),
                               rtol=1e-15)
    # per row, not over the whole array: scaling one row leaves the others
    rng = np.random.default_rng(3)
    X = rng.standard_normal((3, 8))
    w = rng.uniform(0.9, 1.1, 8)
    Y = oracle.head_rmsnorm(X, w, 1e-12)
    X2 = X.copy()
    X2[1] *= 1000.0
    Y2 = oracle.head_rmsnorm(X2, w, 1e-12)
    np.testing.assert_allclose(Y2, Y, rtol=1e-9)         # scale invariance, row by row
    np.testing.assert_allclose(np.sqrt(np.mean((Y / w) ** 2, axis=1)), 1.0, rtol=1e-9)


def test_attn_qgate_reduces_to_plain_attention():
    """With no weights the de-interleaved query goes straight to attn_decode; with a
    key norm the output does not change when the key is scaled (only its direction
    enters), and at position 0 the only key's value is returned whatever the norms."""
    rng = np.random.default_rng(21)
    Hq, Hkv, D, T, pos = 4, 2, 8, 6, 4
    qg = rng.standard_normal((Hq, 2 * D))
    k = rng.standard_normal((Hkv, D))
    v = rng.standard_normal((Hkv, D))
    K = rng.standard_normal((Hkv, T, D))
    V = rng.standard_normal((Hkv, T, D))
    o, gate, K2, V2 = oracle.attn_decode_qgate(qg, k, v, K, V, pos, 1e4, 4)
    o_ref, K_ref, _ = oracle.attn_decode(qg[:, :D], k, v, K, V, pos, 1e4, 4)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(gate, qg[:, D:])
    np.testing.assert_array_equal(K2, K_ref)
    wk = rng.uniform(0.5, 1.5, D)
    wq = rng.uniform(0.5, 1.5, D)
    a = oracle.attn_decode_qgate(qg, k, v, K, V, pos, 1e4, 4, wq, wk, 0.0)
    b = oracle.attn_decode_qgate(qg * 3.0, k * 7.0, v, K, V, pos, 1e4, 4, wq, wk, 0.0)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-12)
    np.testing.assert_allclose(b[2][:, pos], a[2][:, pos], rtol=1e-12)
    # the appended key is the normalised one: its rms over the unrotated dims is |w|
    kn = oracle.head_rmsnorm(k, wk, 0.0)
    np.testing.assert_allclose(a[2][:, pos, 4:], kn[:, 4:], rtol=1e-13)
    o0, _, _, _ = oracle.attn_decode_qgate(qg, k, v, K, V, 0, 1e4, 8, wq, wk, 1e-6)
    np.testing.assert_allclose(o0, np.repeat(v, Hq // Hkv, axis=0), rtol=1e-13)
