"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one part of the oracle to the pages' worked example, a closed
form, a library routine (torch CPU), an invariant the method guarantees, or an
independent brute-force formulation, so that a dropped term, a wrong sign, a
wrong index or a transposed operand fails at least one of them.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("="))
            vals[k] = int(v)
    return vals


def torch_bf16_bits(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_from_bits(u32):
    return np.asarray(u32, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------------------
# bf16 round-to-nearest-even against torch's CPU conversion
# ---------------------------------------------------------------------------
def test_bf16_rne_matches_torch():
    rng = wl.rng_for(11)
    mant = rng.standard_normal(200_000).astype(np.float32)
    expo = rng.integers(-140, 120, size=mant.size).astype(np.float32)
    vals = (mant * np.exp2(expo)).astype(np.float32)
    # exact ties: lower 16 bits == 0x8000, upper half even and odd
    upper = rng.integers(0, 0x7F7F, size=4000).astype(np.uint32)
    ties = f32_from_bits((upper << 16) | 0x8000)
    below = f32_from_bits((upper << 16) | 0x7FFF)
    above = f32_from_bits((upper << 16) | 0x8001)
    edge = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 1e-45, -1e-45, 1.1754942e-38,
                     3.4028235e38, -3.4028235e38, 3.3961776e38, 65504.0, 1.0 / 3.0],
                    dtype=np.float32)
    allv = np.concatenate([vals, ties, -ties, below, above, edge]).astype(np.float32)
    ours = oracle.f32_to_bf16(allv)
    ref = torch_bf16_bits(allv)
    assert np.array_equal(ours, ref)
    nan_in = np.array([np.nan, -np.nan, f32_from_bits(0x7F800001)[()]], dtype=np.float32)
    assert np.isnan(oracle.bf16_to_f32(oracle.f32_to_bf16(nan_in))).all()
    # round trip of every bf16 pattern that is not NaN
    pats = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(pats)
    keep = ~np.isnan(f)
    assert np.array_equal(oracle.f32_to_bf16(f[keep]), pats[keep])


# ---------------------------------------------------------------------------
# Page addressing: the worked block-stride example of the vLLM Ascend page
# ---------------------------------------------------------------------------
def conv_only_geometry(num_slots=6):
    # (W-1) * C = 3 * 16 = 48 bf16 elements per logical block, page 128 bytes
    return wl.Geometry(num_slots=num_slots, C=16, W=4, Hk=0, Hv=0, dk=0, dv=0,
                       page_stride=128, ssm_off=0, conv_off=0)


def numbered_pool(geom):
    el = geom.page_stride // 2
    return np.arange(geom.num_slots * el, dtype=np.uint16).view(np.uint8).reshape(
        geom.num_slots, geom.page_stride).copy()


def test_block_stride_worked_example_gather():
    gold = read_golden("nckv_block_stride.txt")
    g = conv_only_geometry()
    ssm_b, conv_b = oracle.region_bytes(g.C, g.W, g.Hv, g.dk, g.dv)
    assert ssm_b == 0
    assert conv_b == gold["payload_bytes"] == gold["elements_per_block"] * gold["element_bytes"]
    assert g.page_stride == gold["page_bytes"]
    stride = gold["block_stride_elements"]
    assert g.page_stride // gold["element_bytes"] == stride
    pool = numbered_pool(g)
    _, cd = oracle.gather(pool, g, np.arange(g.num_slots))
    for s in range(g.num_slots):
        got = cd[s].view(np.uint16)
        assert np.array_equal(got, np.arange(stride * s, stride * s + gold["elements_per_block"]))


def test_block_stride_worked_example_scatter_and_restore_leave_gap():
    gold = read_golden("nckv_block_stride.txt")
    g = conv_only_geometry()
    n_el = gold["elements_per_block"]
    stride = gold["block_stride_elements"]
    gap = gold["gap_elements"]
    assert n_el + gap == stride
    pool = numbered_pool(g)
    before = pool.copy()
    dense = np.full((2, n_el), 0xFFFF, dtype=np.uint16).view(np.uint8)
    oracle.scatter(pool, g, np.array([1, 4]), np.zeros((2, 0), np.uint8), dense)
    el = pool.view(np.uint16).reshape(-1)
    ref = before.view(np.uint16).reshape(-1).copy()
    for s in (1, 4):
        ref[stride * s: stride * s + n_el] = 0xFFFF
    assert np.array_equal(el, ref)
    # restore of slot 5 into slot 2 moves exactly elements [320, 368) to [128, 176)
    pool = before.copy()
    hs = np.zeros(1, dtype=np.uint8)
    rc = oracle.restore([pool], g, np.array([[2, 5, 1]]), hs)
    assert rc == 0 and hs[0] == 1
    ref = before.view(np.uint16).reshape(-1).copy()
    ref[2 * stride: 2 * stride + n_el] = ref[5 * stride: 5 * stride + n_el]
    assert np.array_equal(pool.view(np.uint16).reshape(-1), ref)


# ---------------------------------------------------------------------------
# Conv + SiLU
# ---------------------------------------------------------------------------
def silu(x):
    return x / (1.0 + np.exp(-x))


@pytest.mark.parametrize("W,bias", [(4, False), (4, True), (2, True), (5, True)])
def test_conv_matches_torch_conv1d(W, bias):
    rng = wl.rng_for(100 + W)
    C, L = 24, 37
    win = wl.to_bf16_bits(rng.standard_normal((W - 1, C), dtype=np.float32))
    x = wl.draw_x(rng, L, C)
    w, b = wl.draw_conv_params(rng, C, W, bias)
    y, new_win = oracle.conv_silu(win, x, w, b)
    seq = np.concatenate([wl.bf16_bits_to_f32(win), wl.bf16_bits_to_f32(x)], axis=0)
    inp = torch.from_numpy(seq.T.astype(np.float64))[None]          # [1, C, W-1+L]
    wt = torch.from_numpy(wl.bf16_bits_to_f32(w).astype(np.float64))[:, None, :]  # [C,1,W]
    bt = None if b is None else torch.from_numpy(wl.bf16_bits_to_f32(b).astype(np.float64))
    ref = F.silu(F.conv1d(inp, wt, bt, groups=C))[0].numpy().T     # [L, C]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # the new window is the last W-1 raw inputs, bit for bit
    full = np.concatenate([win, x], axis=0)
    assert np.array_equal(new_win, full[-(W - 1):])


def test_conv_impulse_response_reads_taps_backwards():
    rng = wl.rng_for(7)
    C, W, L = 8, 4, 7
    w, b = wl.draw_conv_params(rng, C, W, bias=True)
    x = np.zeros((L, C), dtype=np.uint16)
    x[0, :] = wl.to_bf16_bits(np.ones(C, dtype=np.float32))
    y, win = oracle.conv_silu(np.zeros((W - 1, C), np.uint16), x, w, b)
    wf = wl.bf16_bits_to_f32(w).astype(np.float64)
    bf = wl.bf16_bits_to_f32(b).astype(np.float64)
    for t in range(L):
        pre = bf + (wf[:, W - 1 - t] if t < W else 0.0)
        np.testing.assert_allclose(y[t], silu(pre), rtol=1e-14, atol=0)
    assert np.array_equal(win, x[-(W - 1):])


def test_conv_constant_input_ramp():
    rng = wl.rng_for(8)
    C, W, L = 8, 4, 6
    w, b = wl.draw_conv_params(rng, C, W, bias=True)
    a = 0.75
    x = np.tile(wl.to_bf16_bits(np.full(C, a, dtype=np.float32)), (L, 1))
    y, _ = oracle.conv_silu(np.zeros((W - 1, C), np.uint16), x, w, b)
    wf = wl.bf16_bits_to_f32(w).astype(np.float64)
    bf = wl.bf16_bits_to_f32(b).astype(np.float64)
    for t in range(L):
        taps = wf[:, max(0, W - 1 - t):].sum(axis=1)
        np.testing.assert_allclose(y[t], silu(bf + a * taps), rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# Gated delta rule: closed forms
# ---------------------------------------------------------------------------
def unit(v):
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def test_delta_rule_identity_gate_is_plain_readout():
    """alpha=1, beta=0: the state does not move and o = S q (value i = sum_j S[j][i] q_j)."""
    rng = wl.rng_for(21)
    dk, dv, L = 8, 12, 5
    S0 = rng.standard_normal((dk, dv)).astype(np.float32)
    q = rng.standard_normal((L, dk))
    k = unit(rng.standard_normal((L, dk)))
    v = rng.standard_normal((L, dv))
    S, o, _ = oracle.delta_rule(S0, q, k, v, np.ones(L, np.float32), np.zeros(L, np.float32))
    assert np.array_equal(S, S0)
    np.testing.assert_allclose(o, q @ S0.astype(np.float64), rtol=1e-13, atol=1e-13)


def test_delta_rule_full_forget_writes_rank_one():
    """alpha=0: S = beta k v^T (as [key][value]) and o = beta (k.q) v."""
    rng = wl.rng_for(22)
    dk, dv = 8, 12
    S0 = rng.standard_normal((dk, dv)).astype(np.float32)
    q = rng.standard_normal((1, dk))
    k = unit(rng.standard_normal((1, dk)))
    v = rng.standard_normal((1, dv))
    beta = np.array([0.3], np.float32)
    S, o, _ = oracle.delta_rule(S0, q, k, v, np.zeros(1, np.float32), beta)
    b = float(beta[0])
    np.testing.assert_allclose(S, (b * np.outer(k[0], v[0])).astype(np.float32), rtol=1e-6)
    np.testing.assert_allclose(o[0], b * float(k[0] @ q[0]) * v[0], rtol=1e-12)


def test_delta_rule_from_zero_state_single_token():
    rng = wl.rng_for(23)
    dk, dv = 16, 16
    q = rng.standard_normal((1, dk))
    k = unit(rng.standard_normal((1, dk)))
    v = rng.standard_normal((1, dv))
    S, o, _ = oracle.delta_rule(np.zeros((dk, dv), np.float32), q, k, v,
                                np.array([0.37], np.float32), np.array([0.81], np.float32))
    b = float(np.float32(0.81))
    np.testing.assert_allclose(o[0], b * float(k[0] @ q[0]) * v[0], rtol=1e-12)


@pytest.mark.parametrize("alpha", [1.0, 0.5, 0.031])
def test_delta_rule_write_property(alpha):
    """beta=1 and |k|=1: after the update S k = v exactly, whatever alpha and S0
    are -- this fails if the prediction used the undecayed state."""
    rng = wl.rng_for(24)
    dk, dv = 16, 12
    S0 = rng.standard_normal((dk, dv)).astype(np.float32)
    k = unit(rng.standard_normal((1, dk)))
    q = rng.standard_normal((1, dk))
    v = rng.standard_normal((1, dv))
    S, _, _ = oracle.delta_rule(S0, q, k, v, np.array([alpha], np.float32),
                                np.ones(1, np.float32))
    np.testing.assert_allclose(k[0] @ S.astype(np.float64), v[0], rtol=0, atol=2e-6)


def test_delta_rule_orthonormal_keys_store_associations():
    """alpha=beta=1 with orthonormal keys from zero: S = sum_i k_i v_i^T, S k_j = v_j."""
    rng = wl.rng_for(25)
    dk, dv, m = 16, 10, 9
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q[:, :m].T
    vals = rng.standard_normal((m, dv))
    S, _, _ = oracle.delta_rule(np.zeros((dk, dv), np.float32), np.zeros((m, dk)), keys, vals,
                                np.ones(m, np.float32), np.ones(m, np.float32))
    np.testing.assert_allclose(S, keys.T @ vals, atol=2e-6)
    np.testing.assert_allclose(keys @ S.astype(np.float64), vals, atol=5e-6)


def test_delta_rule_pure_decay_over_tokens():
    """beta=0: S_t = (prod alpha) S_0 and o_t = (prod_{s<=t} alpha_s) S_0 q_t."""
    rng = wl.rng_for(26)
    dk, dv, L = 8, 8, 12
    S0 = rng.standard_normal((dk, dv)).astype(np.float32)
    a = rng.uniform(0.5, 1.0, L).astype(np.float32)
    q = rng.standard_normal((L, dk))
    S, o, _ = oracle.delta_rule(S0, q, unit(rng.standard_normal((L, dk))),
                                rng.standard_normal((L, dv)), a, np.zeros(L, np.float32))
    cum = np.cumprod(a.astype(np.float64))
    np.testing.assert_allclose(S, cum[-1] * S0, rtol=1e-5)
    np.testing.assert_allclose(o, cum[:, None] * (q @ S0.astype(np.float64)), rtol=1e-5,
                               atol=1e-6)


def test_delta_rule_bf16_output_is_rne_of_fp32():
    rng = wl.rng_for(27)
    dk, dv, L = 16, 16, 20
    _, o64, o16 = oracle.delta_rule(rng.standard_normal((dk, dv)).astype(np.float32),
                                    rng.standard_normal((L, dk)),
                                    unit(rng.standard_normal((L, dk))),
                                    rng.standard_normal((L, dv)),
                                    rng.uniform(0.1, 1, L).astype(np.float32),
                                    rng.uniform(0, 1, L).astype(np.float32))
    assert np.array_equal(o16, torch_bf16_bits(o64.astype(np.float32)))


# ---------------------------------------------------------------------------
# Whole layer vs an independent product-form formulation (numpy, fp64)
# ---------------------------------------------------------------------------
def product_form_layer(pool, g, inp):
    """Independent restatement: conv via torch conv1d, explicit matrices
    M (value x key) with M_t = a M (I - b k k^T) + b v k^T, o = M q,
    M held as fp32 between tokens; v-head h reads k-head h // (Hv/Hk)."""
    T = inp.total_tokens
    out = np.zeros((T, g.Hv, g.dv))
    G = g.Hv // g.Hk
    wt = torch.from_numpy(wl.bf16_bits_to_f32(inp.conv_w).astype(np.float64))[:, None, :]
    bt = (None if inp.conv_b is None
          else torch.from_numpy(wl.bf16_bits_to_f32(inp.conv_b).astype(np.float64)))
    for n in range(inp.num_seqs):
        t0, t1 = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
        s = int(inp.state_indices[n])
        if t1 == t0 or s < 0 or s >= g.num_slots:
            continue
        page = pool[s]
        if inp.has_initial_state[n]:
            win = page[g.conv_off:g.conv_off + g.conv_region_bytes].view(np.uint16).reshape(
                g.W - 1, g.C).copy()
            st = page[g.ssm_off:g.ssm_off + g.ssm_region_bytes].view(np.float32).reshape(
                g.Hv, g.dk, g.dv).copy()
        else:
            win = np.zeros((g.W - 1, g.C), np.uint16)
            st = np.zeros((g.Hv, g.dk, g.dv), np.float32)
        seq = np.concatenate([win, inp.x[t0:t1]], axis=0)
        xin = torch.from_numpy(wl.bf16_bits_to_f32(seq).T.astype(np.float64))[None]
        y = F.silu(F.conv1d(xin, wt, bt, groups=g.C))[0].numpy().T
        qd = g.Hk * g.dk
        for h in range(g.Hv):
            kh = h // G
            M = st[h].T.astype(np.float64)                    # [dv, dk]
            for t in range(t1 - t0):
                q = y[t, kh * g.dk:(kh + 1) * g.dk]
                k = y[t, qd + kh * g.dk: qd + (kh + 1) * g.dk]
                v = y[t, 2 * qd + h * g.dv: 2 * qd + (h + 1) * g.dv]
                q = inp.scale * q / np.sqrt(q @ q + inp.eps)
                k = k / np.sqrt(k @ k + inp.eps)
                a = float(inp.alpha[t0 + t, h])
                b = float(inp.beta[t0 + t, h])
                M = a * M @ (np.eye(g.dk) - b * np.outer(k, k)) + b * np.outer(v, k)
                out[t0 + t, h] = M @ q
                M = M.astype(np.float32).astype(np.float64)
            st[h] = M.T.astype(np.float32)
        page[g.ssm_off:g.ssm_off + g.ssm_region_bytes] = st.reshape(-1).view(np.uint8)
        page[g.conv_off:g.conv_off + g.conv_region_bytes] = (
            seq[-(g.W - 1):].reshape(-1).view(np.uint8))
    return out


def layer_case(g, seed, lengths, warm, bias=False, scale=1.0, long_memory=False, eps=1e-6):
    rng = wl.rng_for(seed)
    n = len(lengths)
    idx = rng.permutation(g.num_slots)[:n].astype(np.int32)
    hs = np.asarray(warm, dtype=np.uint8)
    img = wl.make_pool_image(g, rng, warm_slots=idx[hs == 1], nan_slots=idx[hs == 0],
                             sigma_s=0.5)
    inp = wl.step_inputs(g, rng, lengths, idx, hs, bias=bias, long_memory=long_memory)
    inp.scale = scale
    inp.eps = eps
    return inp, img


def run_oracle(img, inp):
    return oracle.gdn_layer(img, inp.geom, inp.cu_seqlens, inp.state_indices,
                            inp.has_initial_state, inp.x, inp.conv_w, inp.conv_b, inp.alpha,
                            inp.beta, inp.scale, inp.eps)


@pytest.mark.parametrize("Hk,Hv,dk,dv,bias,scale,eps", [
    (1, 2, 16, 16, False, 1.0, 1e-6),
    (1, 2, 16, 16, True, 0.25, 1e-6),
    (2, 4, 8, 8, True, 1.0, 1e-6),     # two k-heads: pins the v-head -> k-head mapping
    (2, 2, 8, 12, False, 0.5, 1e-6),   # dk != dv: pins which index is the key
    (1, 2, 8, 8, True, 1.0, 0.5),      # eps comparable to |k|^2: pins where eps enters
])
def test_layer_matches_product_form(Hk, Hv, dk, dv, bias, scale, eps):
    g = wl.make_geometry(8, Hk=Hk, Hv=Hv, dk=dk, dv=dv, W=4, page_align=128, extra_pad=128)
    inp, img = layer_case(g, 31, [19, 1, 7, 12], [1, 0, 1, 0], bias=bias, scale=scale, eps=eps)
    ref_pool = img.copy()
    o64, o16 = run_oracle(img, inp)
    ref = product_form_layer(ref_pool, g, inp)
    scale_o = np.abs(ref).max()
    assert scale_o > 1e-3
    # both sides are fp64 and differ only in rounding order: ~1e-13 element-wise
    np.testing.assert_allclose(o64, ref, rtol=1e-12, atol=1e-14 * scale_o)
    assert np.array_equal(o16, torch_bf16_bits(o64.astype(np.float32)))
    # windows, padding and the fp32 state words bit-exact (the two fp64 forms
    # land on the same fp32 rounding of every state entry)
    for s in range(g.num_slots):
        a, b = img[s], ref_pool[s]
        cw = slice(g.conv_off, g.conv_off + g.conv_region_bytes)
        assert np.array_equal(a[cw], b[cw])
        pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
        assert np.array_equal(a[pad], b[pad])
        sa = a[g.ssm_off:g.ssm_off + g.ssm_region_bytes].view(np.uint32)
        sb = b[g.ssm_off:g.ssm_off + g.ssm_region_bytes].view(np.uint32)
        assert np.array_equal(sa, sb)
