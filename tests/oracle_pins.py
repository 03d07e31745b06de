"""Checks that pin the CPU oracle to facts that do not come from the oracle itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with what the
pages or the mathematics fix: the exact-equivalence claim of QK-Normed MLA
(explicit post-projection QK RMSNorm equals the absorbed latent form), closed
forms on hand-built inputs, invariants of attention, and library routines
(torch's bfloat16 conversion, ``rms_norm`` and ``scaled_dot_product_attention``).
They are plain functions so that tests/test_oracle_mutations.py can plant
mistakes in the oracle and confirm that some check catches each of them.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import workloads as W
from oracle import qkn_oracle as O


def small(name, **kw):
    """The named workload at a size the float64 oracle finishes in well under a second."""
    base = {
        "tiny": dict(),
        "dsv3": dict(batch=2, seq_len=200),
        "grouped": dict(batch=2, seq_len=150),
        "long": dict(batch=1, seq_len=1000, num_splits=7),
        "mtp": dict(batch=3, seq_len=200, seq_len_range=(5, 200)),
    }[name]
    base.update(kw)
    return W.WORKLOADS[name].replace(**base)


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# encodings and building blocks against library routines
# ---------------------------------------------------------------------------

def check_bf16_against_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    bits = x.view(np.uint32)
    # exact ties (low half = 0x8000) with even and odd kept lsb, and near-ties
    ties = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    near = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-40, -1e-42,
                         1.17549435e-38, 65504.0, 1.0, -1.0], dtype=np.float32)
    allx = np.concatenate([x, ties.view(np.float32), near.view(np.float32), specials])
    ours = O.f32_to_bf16_bits(allx)
    ref = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref), "bf16 RNE differs from torch"
    nan = np.array([np.nan], dtype=np.float32)
    assert np.isnan(O.bf16_bits_to_f32(O.f32_to_bf16_bits(nan)))[0]
    back = O.bf16_bits_to_f32(ours)
    ref_back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back, ref_back)


def check_f16_against_torch():
    """The half storage words against torch's float32 -> float16 cast (IEEE
    round to nearest even), ties, subnormals, overflow to inf and signed zero."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(5.0)
    tiny = rng.standard_normal(1000).astype(np.float32) * np.float32(1e-6)   # subnormal halves
    ties = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 65504.0,
                     65519.0, 65520.0, 1e6, -0.0, 0.0, -1e-9], dtype=np.float32)
    for v in (x, tiny, ties):
        got = O.stored_bits(v.astype(np.float64), "f16")
        want = torch.from_numpy(v).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want)
        back = O.words_to_f64(got, "f16")
        assert np.array_equal(back, torch.from_numpy(v).to(torch.float16).double().numpy())


def check_rmsnorm_against_torch():
    rng = np.random.default_rng(2)
    for eps in (1e-6, 0.5, 3.0):
        z = rng.standard_normal((17, 128)) * 0.3
        g = 1 + 0.1 * rng.standard_normal(128)
        ours = O.rmsnorm(z, g, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(z), (128,), torch.from_numpy(g), eps)
        assert np.allclose(ours, ref.numpy(), rtol=1e-13, atol=0), f"rms_norm differs at eps={eps}"
        # the scalar form alpha = 1/S(z) against the same routine with unit weight
        ones = torch.nn.functional.rms_norm(torch.from_numpy(z), (128,), None, eps).numpy()
        assert np.allclose(O.inv_rms(z, eps)[:, None] * z, ones, rtol=1e-13, atol=0)


def check_rope_properties():
    rng = np.random.default_rng(3)
    for dR in (2, 16, 64):
        x = rng.standard_normal((5, dR))
        y = rng.standard_normal((5, dR))
        # position 0 is the identity
        assert np.allclose(O.rope(x, 0, 10000.0), x, rtol=0, atol=0)
        for pos in (1, 7, 4095, 262143):
            rx = O.rope(x, pos, 10000.0)
            # a rotation keeps lengths
            assert np.allclose(np.linalg.norm(rx, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
        # scores depend only on the relative position
        for m, n in ((5, 3), (1000, 12), (70000, 69990)):
            lhs = np.sum(O.rope(x, m, 10000.0) * O.rope(y, n, 10000.0), axis=-1)
            rhs = np.sum(O.rope(x, m - n, 10000.0) * y, axis=-1)
            assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-9)
        # rotating by a then b equals rotating by a + b
        assert np.allclose(O.rope(O.rope(x, 11, 10000.0), 31, 10000.0), O.rope(x, 42, 10000.0),
                           rtol=1e-12, atol=1e-12)
    # d_R = 2: one pair at frequency theta^0 = 1, i.e. the complex number a + ib times e^{i pos}
    for pos in (0, 1, 3, 100):
        a, b = 0.3, -1.7
        z = complex(a, b) * complex(math.cos(pos), math.sin(pos))
        got = O.rope(np.array([a, b]), pos, 10000.0)
        assert np.allclose(got, [z.real, z.imag], rtol=1e-13, atol=1e-13)
    # theta 0 disables the rotation
    x = rng.standard_normal((3, 8))
    assert np.array_equal(O.rope(x, 99, 0.0), x)


def check_rope_frequency_ladder():
    """Every pair's frequency, not only the first: against the rotary embedding
    of the transformers library (Llama's default rotary parameters, NeoX
    rotate-half pairs (j, j + d_R/2)), and against angles worked out by hand.

    The library computes its angles in float32, so positions stay small
    (angle error ~1e-6) while a wrong ladder moves some angle by O(1)."""
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as ML

    rng = np.random.default_rng(30)
    for dR in (4, 8, 16, 64):
        cfg = LlamaConfig(hidden_size=4 * dR, num_attention_heads=4, head_dim=dR,
                          rope_theta=10000.0)
        emb = ML.LlamaRotaryEmbedding(cfg)
        pos = np.array([0, 1, 2, 3, 7, 13, 31, 50], dtype=np.int64)
        x = rng.standard_normal((1, 1, len(pos), dR))
        cos, sin = emb(torch.from_numpy(x), torch.from_numpy(pos)[None, :])
        ref, _ = ML.apply_rotary_pos_emb(torch.from_numpy(x), torch.from_numpy(x), cos, sin)
        got = O.rope(x[0, 0], pos, 10000.0)
        assert np.allclose(got, ref[0, 0].numpy(), rtol=0, atol=2e-5), \
            f"d_R={dR}: RoPE differs from the library by {np.max(np.abs(got - ref[0, 0].numpy()))}"
    # Hand-worked angles at theta = 10000: the pair j of a d_R-wide block turns
    # at 10000^(-2j/d_R) radians per position, so
    #   d_R = 4, j = 1: 10^-2  -> position 100 turns it by exactly 1 rad;
    #   d_R = 8, j = 1: 10^-1  -> position 10 gives 1 rad; j = 3: 10^-3 -> position 1000.
    for dR, j, pos in ((4, 1, 100), (8, 1, 10), (8, 2, 100), (8, 3, 1000), (16, 4, 100)):
        half = dR // 2
        e = np.zeros(dR)
        e[j] = 1.0
        got = O.rope(e, pos, 10000.0)
        want = np.zeros(dR)
        want[j], want[j + half] = math.cos(1.0), math.sin(1.0)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (dR, j, pos, got)
        # the partner coordinate turns the other way round
        e2 = np.zeros(dR)
        e2[j + half] = 1.0
        want2 = np.zeros(dR)
        want2[j], want2[j + half] = -math.sin(1.0), math.cos(1.0)
        assert np.allclose(O.rope(e2, pos, 10000.0), want2, rtol=0, atol=1e-12)


def check_value_up_projection(name):
    """The value side of the absorbed path, o = o^lat W^V_g, against the explicit
    path's o = sum_t p_t (c_t W^V_g) with the values materialised: equal by
    linearity, to float64 rounding, for every head of every group."""
    wl = small(name)
    inp = W.make_inputs(wl, seed=31)
    heads = np.arange(wl.heads)
    worst = 0.0
    for b in range(wl.batch):
        for i in range(wl.s_q):
            e = O.explicit_rows(wl, inp, b, i)
            o = O.value_up_projection(wl, e["o_lat"], inp["w_v"], heads)
            worst = max(worst, rel_err(o, e["o"]))
            # a subset of heads, out of order, maps each head to its own group
            sub = heads[::-7]
            o_sub = O.value_up_projection(wl, e["o_lat"][sub], inp["w_v"], sub)
            worst = max(worst, rel_err(o_sub, e["o"][sub]))
    assert worst <= 1e-10, f"{name}: value up-projection vs explicit values {worst:.3e}"
    return worst


# ---------------------------------------------------------------------------
# the method: exact equivalence and closed forms
# ---------------------------------------------------------------------------

def check_explicit_equals_absorbed(name, tol=1e-10):
    wl = small(name)
    inp = W.make_inputs(wl, seed=0)
    worst = 0.0
    for b in range(wl.batch):
        for i in range(wl.s_q):
            e = O.explicit_rows(wl, inp, b, i)
            a = O.absorbed_rows(wl, inp, b, i)
            worst = max(worst, rel_err(a["o"], e["o"]), rel_err(a["o_lat"], e["o_lat"]),
                        rel_err(a["lse"], e["lse"]))
    assert worst <= tol, f"{name}: explicit vs absorbed rel err {worst:.3e}"
    return worst


def check_rows_sum_to_one(name):
    wl = small(name)
    inp = W.make_inputs(wl, seed=4)
    inp["c"][:, 0] = 1.0
    for b in range(wl.batch):
        for i in range(wl.s_q):
            e = O.explicit_rows(wl, inp, b, i)
            assert np.allclose(e["p"].sum(-1), 1.0, rtol=0, atol=1e-12)
            assert np.allclose(e["o_lat"][:, 0], 1.0, rtol=0, atol=1e-12)
            a = O.absorbed_rows(wl, inp, b, i)
            assert np.allclose(a["o_lat"][:, 0], 1.0, rtol=0, atol=1e-12)


def check_single_token():
    """T = 1: the only visible token gets all the weight; lse equals its logit."""
    wl = W.WORKLOADS["tiny"].replace(seq_len=1)
    inp = W.make_inputs(wl, seed=5)
    e = O.explicit_rows(wl, inp, 0, 0)
    a = O.absorbed_rows(wl, inp, 0, 0)
    c0 = inp["c"][0].astype(np.float64)
    assert np.allclose(e["o_lat"], c0[None, :], rtol=1e-15, atol=0)
    assert np.allclose(a["o_lat"], c0[None, :], rtol=1e-14, atol=0)
    assert np.allclose(e["o"], (c0 @ inp["w_v"][0].astype(np.float64))[None, :], rtol=1e-13, atol=1e-15)


def _geometric_case(scale_c=(3.0, -0.5, 2.0), eps=0.0):
    """Hand-built inputs whose normalised dot products are known exactly.

    r = d = 4, W^K = W^V = I, unit norm weights, no RoPE block, eps = 0.
    Keys: c_0 = 3 e_0, c_1 = -0.5 e_0, c_2 = 2 e_1  ->  k^_0 = 2 e_0, k^_1 = -2 e_0,
    k^_2 = 2 e_1 (a unit-weight RMSNorm of s e_j is sign(s) sqrt(d) e_j).
    Queries: head 0 along e_0, head 1 along e_1 (any positive length)."""
    d = 4
    wl = W.Workload("geo", batch=1, s_q=1, heads=2, groups=1, rank=d, head_dim=d, rope_dim=0,
                    seq_len=3, cache_dtype="f32", latent_log_sigma=0.0, num_splits=1, eps=eps)
    c = np.zeros((3, d), np.float32)
    c[0, 0], c[1, 0], c[2, 1] = scale_c
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, 0, 0] = 0.7
    q[0, 0, 1, 1] = 5.0
    inp = {
        "w_k": np.eye(d, dtype=np.float32)[None], "w_v": np.eye(d, dtype=np.float32)[None],
        "gamma_q": np.ones(d, np.float32), "gamma_k": np.ones((1, d), np.float32),
        "gamma_qr": np.ones(0, np.float32), "gamma_kr": np.ones(0, np.float32),
        "seq_lens": np.array([3], np.int32), "tok_offsets": np.array([0, 3]),
        "c": c, "k_rope": np.zeros((3, 0), np.float32), "q": q,
        "q_rope": np.zeros((1, 1, 2, 0), np.float32),
        "block_table": np.array([[0]], np.int32), "num_pages": 1,
    }
    return wl, inp


def check_geometric_closed_form():
    wl, inp = _geometric_case()
    s = wl.softmax_scale  # 1/sqrt(4) = 0.5
    d = 4
    # q^ . k^ = d * cos(angle): head 0 sees [+d, -d, 0], head 1 sees [0, 0, +d]
    l0 = np.array([s * d, -s * d, 0.0])
    l1 = np.array([0.0, 0.0, s * d])
    p0 = np.exp(l0) / np.exp(l0).sum()
    p1 = np.exp(l1) / np.exp(l1).sum()
    c = inp["c"].astype(np.float64)
    for path in (O.explicit_rows, O.absorbed_rows):
        res = path(wl, inp, 0, 0)
        assert np.allclose(res["o_lat"][0], p0 @ c, rtol=1e-14, atol=1e-15)
        assert np.allclose(res["o_lat"][1], p1 @ c, rtol=1e-14, atol=1e-15)
        assert np.allclose(res["lse"], [np.log(np.exp(l0).sum()), np.log(np.exp(l1).sum())],
                           rtol=1e-14)
    # two visible tokens: p_0 = sigmoid(l_0 - l_1)
    wl2 = wl.replace(seq_len=2)
    inp2 = dict(inp, seq_lens=np.array([2], np.int32), tok_offsets=np.array([0, 2]),
                c=inp["c"][:2], k_rope=inp["k_rope"][:2])
    res = O.explicit_rows(wl2, inp2, 0, 0)
    assert abs(res["p"][0, 0] - 1.0 / (1.0 + math.exp(-(2 * s * d)))) < 1e-15


def check_scale_invariance():
    """With eps = 0 the normalised logits ignore any positive rescaling of a
    latent (the purpose of QK-norm); negative scales flip the key."""
    wl = small("dsv3", batch=1, seq_len=70).replace(eps=0.0)
    inp = W.make_inputs(wl, seed=6)
    base = O.explicit_rows(wl, inp, 0, 0)
    rng = np.random.default_rng(7)
    inp2 = dict(inp)
    # powers of two keep the scaled latents exact in float32
    lam = np.exp2(rng.integers(-20, 21, size=(inp["c"].shape[0], 1))).astype(np.float32)
    inp2["c"] = (inp["c"] * lam).astype(np.float32)
    scaled = O.explicit_rows(wl, inp2, 0, 0)
    assert np.allclose(scaled["p"], base["p"], rtol=1e-9, atol=1e-15)
    assert np.allclose(scaled["lse"], base["lse"], rtol=1e-11)
    a2 = O.absorbed_rows(wl, inp2, 0, 0)
    assert np.allclose(a2["lse"], base["lse"], rtol=1e-10)


def check_bounded_logits():
    """|q^ . k^| <= d * max|gamma_q| * max|gamma_k| (Cauchy-Schwarz on vectors of
    RMS 1 scaled by the weights), however large the raw activations are."""
    wl = small("dsv3", batch=1, seq_len=64).replace(rope_dim=0)
    inp = W.make_inputs(wl, seed=8)
    inp["c"] = inp["c"] * np.float32(1e15)
    inp["q"] = inp["q"] * np.float32(1e12)
    e = O.explicit_rows(wl, inp, 0, 0)
    logits = e["lse"][:, None] + np.log(e["p"])
    bound = wl.softmax_scale * wl.head_dim * np.max(np.abs(inp["gamma_q"])) * np.max(np.abs(inp["gamma_k"]))
    assert np.all(np.abs(logits) <= bound * (1 + 1e-12))


def check_textbook_reduction():
    """r = d, W^K = W^V = I, unit weights, one group, no RoPE block: the method is
    per-head QK-RMSNorm attention; compare with torch's rms_norm and
    scaled_dot_product_attention (causal mask for s_q > 1)."""
    for s_q in (1, 3):
        d = 16
        wl = W.Workload("tb", batch=2, s_q=s_q, heads=4, groups=1, rank=d, head_dim=d, rope_dim=0,
                        seq_len=37, cache_dtype="f32", latent_log_sigma=0.7, num_splits=1)
        inp = W.make_inputs(wl, seed=9)
        inp["w_k"] = np.eye(d, dtype=np.float32)[None]
        inp["w_v"] = np.eye(d, dtype=np.float32)[None]
        inp["gamma_q"] = np.ones(d, np.float32)
        inp["gamma_k"] = np.ones((1, d), np.float32)
        for b in range(wl.batch):
            T = int(inp["seq_lens"][b])
            C = torch.from_numpy(inp["c"][inp["tok_offsets"][b]:inp["tok_offsets"][b + 1]]).double()
            q = torch.from_numpy(inp["q"][b]).double()                     # [s_q, H, d]
            qn = torch.nn.functional.rms_norm(q, (d,), None, wl.eps).permute(1, 0, 2)   # [H, s_q, d]
            kn = torch.nn.functional.rms_norm(C, (d,), None, wl.eps)
            mask = torch.zeros((s_q, T), dtype=torch.bool)
            for i in range(s_q):
                mask[i, :T - s_q + i + 1] = True
            ref = torch.nn.functional.scaled_dot_product_attention(
                qn, kn.expand(wl.heads, T, d).contiguous(), C.expand(wl.heads, T, d).contiguous(),
                attn_mask=mask, scale=wl.softmax_scale)                    # [H, s_q, d]
            for i in range(s_q):
                e = O.explicit_rows(wl, inp, b, i)
                assert np.allclose(e["o"], ref[:, i].numpy(), rtol=1e-12, atol=1e-13)
                assert np.allclose(e["o_lat"], ref[:, i].numpy(), rtol=1e-12, atol=1e-13)


def check_causal_prefix():
    """Query i of a multi-token step equals a single-token step on the prefix of
    length T - s_q + i + 1 whose last token is that query's own position."""
    wl = small("mtp", batch=2)
    inp = W.make_inputs(wl, seed=10)
    wl1 = wl.replace(s_q=1, seq_len_range=None)
    for b in range(wl.batch):
        T = int(inp["seq_lens"][b])
        for i in range(wl.s_q):
            full = O.explicit_rows(wl, inp, b, i)
            n = T - wl.s_q + i + 1
            o0 = inp["tok_offsets"][b]
            sub = dict(inp, seq_lens=np.array([n], np.int32), tok_offsets=np.array([0, n]),
                       c=inp["c"][o0:o0 + n], k_rope=inp["k_rope"][o0:o0 + n],
                       q=inp["q"][b:b + 1, i:i + 1], q_rope=inp["q_rope"][b:b + 1, i:i + 1])
            one = O.explicit_rows(wl1.replace(batch=1, seq_len=n), sub, 0, 0)
            assert np.allclose(full["o_lat"], one["o_lat"], rtol=1e-13, atol=1e-14)
            assert np.allclose(full["lse"], one["lse"], rtol=1e-13)


def check_group_collapse():
    """G = 4 groups with identical up-projections and key weights equals G = 1."""
    wl4 = small("grouped", batch=1, seq_len=90)
    inp = W.make_inputs(wl4, seed=11)
    for k in ("w_k", "w_v", "gamma_k"):
        inp[k] = np.repeat(inp[k][:1], 4, axis=0)
    wl1 = wl4.replace(groups=1)
    inp1 = dict(inp, w_k=inp["w_k"][:1], w_v=inp["w_v"][:1], gamma_k=inp["gamma_k"][:1])
    a = O.explicit_rows(wl4, inp, 0, 0)
    b = O.explicit_rows(wl1, inp1, 0, 0)
    assert np.allclose(a["o"], b["o"], rtol=1e-14, atol=1e-15)
    assert np.allclose(a["lse"], b["lse"], rtol=1e-14)


# ---------------------------------------------------------------------------
# storage images, paging, split-KV
# ---------------------------------------------------------------------------

def check_cache_image_layout():
    wl = small("mtp", batch=3)
    inp = W.make_inputs(wl, seed=12, extra_pages=3)
    kv0, ak0 = O.empty_images(wl, inp["num_pages"])
    img = O.full_cache_image(wl, inp, kv0, ak0)
    kv, ak = img["kv"], img["alpha_k"]
    bt = inp["block_table"]
    ref_bits = torch.from_numpy(inp["c"]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    written = np.zeros(kv.shape[:2], bool)
    for b in range(wl.batch):
        for t in range(int(inp["seq_lens"][b])):
            pg, sl = bt[b, t // 64], t % 64
            assert np.array_equal(kv[pg, sl, :wl.rank], ref_bits[inp["tok_offsets"][b] + t])
            written[pg, sl] = True
    assert np.all(kv[~written] == 0x7FC1) and np.all(np.isnan(ak[~written]))
    assert np.all(np.isfinite(ak[written])) and np.all(ak[written] > 0)


def check_image_decode_matches_explicit_f32():
    """With an fp32 cache the stored state differs from the inputs only by float32
    rounding of q~, alpha and the normed RoPE vectors, so the decode over the
    stored, paged state must agree with the explicit float64 path to ~1e-6."""
    for name in ("tiny", "mtp"):
        wl = small(name).replace(cache_dtype="f32")
        inp = W.make_inputs(wl, seed=13)
        img = O.full_cache_image(wl, inp)
        qi = O.query_image(wl, inp)
        res = O.decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                inp["seq_lens"], num_splits=3)
        for b in range(wl.batch):
            for i in range(wl.s_q):
                e = O.explicit_rows(wl, inp, b, i)
                got = np.stack([res[(b, i, h)]["o_lat"] for h in range(wl.heads)])
                lse = np.array([res[(b, i, h)]["lse"] for h in range(wl.heads)])
                assert rel_err(got, e["o_lat"]) < 2e-5, rel_err(got, e["o_lat"])
                assert np.max(np.abs(lse - e["lse"])) < 2e-5


def check_bf16_image_within_tolerance():
    """The bf16 storage alone (before any kernel) stays well inside the 1e-2
    end-to-end budget against the explicit float64 path."""
    wl = small("dsv3", batch=1, seq_len=300)
    inp = W.make_inputs(wl, seed=14)
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    res = O.decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                            inp["seq_lens"], num_splits=2)
    e = O.explicit_rows(wl, inp, 0, 0)
    got = np.stack([res[(0, 0, h)]["o_lat"] for h in range(wl.heads)])
    rowerr = np.max(np.abs(got - e["o_lat"]), axis=1) / np.max(np.abs(e["o_lat"]), axis=1)
    # about half of the 1e-2 budget goes to rounding c_t and q~ to bf16
    assert np.max(rowerr) < 7.5e-3, np.max(rowerr)
    return float(np.max(rowerr))


def check_split_invariance():
    wl = small("long", seq_len=1000)
    inp = W.make_inputs(wl, seed=15)
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    rows = [(0, 0, h) for h in (0, 5, 77, 127)]
    ref = O.decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                            inp["seq_lens"], num_splits=1, rows=rows)
    for P in (2, 7, 16, 40):   # 40 splits leaves empty partitions (16 pages only)
        got = O.decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                inp["seq_lens"], num_splits=P, rows=rows)
        for k in rows:
            assert np.allclose(got[k]["o_lat"], ref[k]["o_lat"], rtol=1e-12, atol=1e-13)
            assert abs(got[k]["lse"] - ref[k]["lse"]) < 1e-12
            if P == 40:
                assert np.isneginf(got[k]["lse_part"][-1]) and not np.any(got[k]["o_part"][-1])


def check_split_bounds():
    # splits are whole pages, cover [0, T) in order without overlap
    for T in (1, 63, 64, 65, 1000, 4096, 262144, 8191):
        for P in (1, 2, 3, 8, 64, 256):
            bounds = O.split_bounds(T, P)
            assert bounds[0][0] == 0 and bounds[-1][1] == T and len(bounds) == P
            for (a, b), (c, _) in zip(bounds, bounds[1:]):
                assert b == c and a <= b
            for (a, b) in bounds:
                assert a % 64 == 0 or a == T
            lens = [b - a for a, b in bounds]
            assert max(lens) <= -(-T // P) + 63


def check_page_permutation():
    wl = small("dsv3", batch=2, seq_len=333)
    inp = W.make_inputs(wl, seed=16)
    inp2 = W.permute_pages(inp, seed=17)
    qi = O.query_image(wl, inp)
    a = O.full_cache_image(wl, inp)
    b = O.full_cache_image(wl, inp2)
    rows = [(0, 0, 3), (1, 0, 100)]
    ra = O.decode_on_image(wl, qi, a["kv"], a["alpha_k"], inp["block_table"], inp["seq_lens"], 3, rows)
    rb = O.decode_on_image(wl, qi, b["kv"], b["alpha_k"], inp2["block_table"], inp2["seq_lens"], 3, rows)
    for k in rows:
        assert np.array_equal(ra[k]["o_lat"], rb[k]["o_lat"])


def check_combine_closed_form():
    # two splits holding one token each: weights are softmax of the two lse values
    o = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    lse = np.array([[0.3, -1.2]])
    got, l = O.combine(o, lse)
    w0 = 1.0 / (1.0 + math.exp(-1.5))
    assert np.allclose(got, [[w0, 1 - w0]], rtol=1e-15)
    assert abs(l[0] - math.log(math.exp(0.3) + math.exp(-1.2))) < 1e-15
    # an empty split (-inf) changes nothing
    got2, l2 = O.combine(np.concatenate([o, np.full((1, 1, 2), 0.0)], 1),
                         np.concatenate([lse, [[-np.inf]]], 1))
    assert np.allclose(got2, got, rtol=0, atol=0) and l2[0] == l[0]


def check_no_alpha_is_plain_mla():
    """With unit norm weights and the inverse-RMS factors dropped, the decode over
    the stored state is plain absorbed MLA: logits scale * (q~ . c + q^R . k^R)
    with q~ = q W^K^T; compare with explicit un-normalised MLA attention."""
    wl = small("dsv3", batch=1, seq_len=130).replace(cache_dtype="f32", rope_theta=0.0)
    inp = W.make_inputs(wl, seed=18)
    d, dR = wl.head_dim, wl.rope_dim
    inp["gamma_q"] = np.ones(d, np.float32)
    inp["gamma_k"] = np.ones((1, d), np.float32)
    inp["gamma_qr"] = np.ones(dR, np.float32)
    inp["gamma_kr"] = np.ones(dR, np.float32)
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    res = O.decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"], inp["seq_lens"],
                            num_splits=1, use_alpha=False)
    # explicit un-normalised MLA (RoPE block still RMS-normed as stored)
    C = inp["c"].astype(np.float64)
    K = C @ inp["w_k"][0].astype(np.float64)
    q = inp["q"][0, 0].astype(np.float64)
    kr = O.rmsnorm(inp["k_rope"], inp["gamma_kr"], wl.eps)
    qr = O.rmsnorm(inp["q_rope"][0, 0], inp["gamma_qr"], wl.eps)
    logits = wl.softmax_scale * (q @ K.T + qr @ kr.T)
    p = np.exp(logits - logits.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    ref = p @ C
    got = np.stack([res[(0, 0, h)]["o_lat"] for h in range(wl.heads)])
    assert rel_err(got, ref) < 1e-5


# ---------------------------------------------------------------------------
# sparse (selected-token) decode
# ---------------------------------------------------------------------------

def _visible_lists(wl, inp, K):
    """Per (b, i): every visible position in order, padded with -1 to K entries."""
    idx = np.full((wl.batch, wl.s_q, K), -1, dtype=np.int32)
    for b, T in enumerate(inp["seq_lens"]):
        for i in range(wl.s_q):
            n = O.visible_count(int(T), wl.s_q, i)
            idx[b, i, :n] = np.arange(n)
    return idx


def check_sparse_split_bounds():
    # runs of whole 32-entry stages that cover [0, K) in order
    for K in (1, 31, 32, 33, 100, 2048, 2049):
        for Pn in (1, 2, 3, 8, 64):
            bounds = O.sparse_split_bounds(K, Pn)
            assert bounds[0][0] == 0 and bounds[-1][1] == K and len(bounds) == Pn
            for (a, b), (c, _) in zip(bounds, bounds[1:]):
                assert b == c and a <= b
            for (a, b) in bounds:
                assert a % 32 == 0 or a == K
            assert max(b - a for a, b in bounds) <= -(-K // Pn) + 31


def check_sparse_all_visible_equals_dense(name):
    """Listing every visible token gives the dense decode's merged result (the
    split structure differs, the merged softmax does not)."""
    wl = small(name)
    inp = W.make_inputs(wl, seed=33)
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    K = int(np.max(inp["seq_lens"])) + 5
    idx = _visible_lists(wl, inp, K)
    dense = O.decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                              inp["seq_lens"], num_splits=2)
    for Pn in (1, 3):
        sp, err = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                           inp["seq_lens"], idx, Pn)
        assert not err
        for k, v in dense.items():
            assert np.allclose(sp[k]["o_lat"], v["o_lat"], rtol=1e-12, atol=1e-13)
            assert abs(sp[k]["lse"] - v["lse"]) < 1e-12


def check_sparse_subset_against_explicit():
    """A subset S of the visible tokens, against the explicit float64 path:
    restricting its softmax to S gives o^lat = sum_S p_t c_t / sum_S p_t and
    lse = lse_all + ln sum_S p_t.  With an fp32 cache the stored state differs
    from the inputs only by float32 rounding (tolerance as for the dense
    decode).  Also: order, -1 padding and split count leave the result as is;
    a list with one valid entry gives that token's latent exactly."""
    wl = small("mtp").replace(cache_dtype="f32")
    inp = W.make_inputs(wl, seed=34)
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    rng = np.random.default_rng(35)
    K = 96
    idx = np.full((wl.batch, wl.s_q, K), -1, dtype=np.int32)
    subsets = {}
    for b, T in enumerate(inp["seq_lens"]):
        for i in range(wl.s_q):
            n = O.visible_count(int(T), wl.s_q, i)
            m = min(n, int(rng.integers(1, 60)))
            S = rng.choice(n, size=m, replace=False)
            subsets[(b, i)] = np.sort(S)
            slots = np.sort(rng.choice(K, size=m, replace=False))
            idx[b, i, slots] = S
    sp, err = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                       inp["seq_lens"], idx, 3)
    assert not err
    for (b, i), S in subsets.items():
        e = O.explicit_rows(wl, inp, b, i)
        C = np.asarray(inp["c"][inp["tok_offsets"][b] + S], dtype=np.float64)
        w = e["p"][:, S]
        want = (w @ C) / w.sum(axis=1, keepdims=True)
        want_lse = e["lse"] + np.log(w.sum(axis=1))
        got = np.stack([sp[(b, i, h)]["o_lat"] for h in range(wl.heads)])
        lse = np.array([sp[(b, i, h)]["lse"] for h in range(wl.heads)])
        assert rel_err(got, want) < 2e-5, rel_err(got, want)
        assert np.max(np.abs(lse - want_lse)) < 2e-5
    # order, padding and split count do not matter
    perm = idx[..., ::-1].copy()
    pad = np.concatenate([np.full(idx.shape[:2] + (40,), -1, np.int32), idx], axis=2)
    for alt, Pn in ((perm, 3), (pad, 1), (idx, 5)):
        sp2, _ = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                          inp["seq_lens"], alt, Pn)
        for k, v in sp.items():
            assert np.allclose(sp2[k]["o_lat"], v["o_lat"], rtol=1e-12, atol=1e-13)
            assert abs(sp2[k]["lse"] - v["lse"]) < 1e-12
    # one valid entry: o^lat is that latent as stored, lse its logit
    one = np.full((wl.batch, wl.s_q, 40), -1, dtype=np.int32)
    one[:, :, 17] = 2
    sp1, _ = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                      inp["seq_lens"], one, 2)
    for b in range(wl.batch):
        e = O.explicit_rows(wl, inp, b, 0)
        page = inp["block_table"][b, 0]
        c2 = O.words_to_f64(img["kv"][page, 2, :wl.rank], "f32")
        for h in range(wl.heads):
            assert np.array_equal(sp1[(b, 0, h)]["o_lat"], c2)
            assert abs(sp1[(b, 0, h)]["lse"] - (e["lse"][h] + np.log(e["p"][h, 2]))) < 2e-5


def check_sparse_invalid_entries():
    """Entries past the visible end, below -1, or on an out-of-range page entry
    are reported and ignored; a list of -1 only is the empty sum (o = 0,
    lse = -inf) and is not an error."""
    wl = small("dsv3")
    inp = W.make_inputs(wl, seed=36)
    img = O.full_cache_image(wl, inp)
    qi = O.query_image(wl, inp)
    base = np.full((wl.batch, 1, 64), -1, dtype=np.int32)
    base[:, 0, :5] = [0, 9, 33, 64, 101]
    ref, err = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                        inp["seq_lens"], base, 2)
    assert not err
    bad = base.copy()
    bad[:, 0, 20] = int(inp["seq_lens"][0]) + 3   # past the visible end
    bad[:, 0, 40] = -7
    got, err = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                        inp["seq_lens"], bad, 2)
    assert err
    for k, v in ref.items():
        assert np.array_equal(got[k]["o_lat"], v["o_lat"]) and got[k]["lse"] == v["lse"]
    bt = inp["block_table"].copy()
    bt[:, 1] = img["kv"].shape[0] + 4               # page of positions 64 .. 127 out of range
    got, err = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], bt,
                                        inp["seq_lens"], base, 2)
    assert err
    drop = base.copy()
    drop[:, 0, 3:5] = -1
    want, _ = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                       inp["seq_lens"], drop, 2)
    for k, v in want.items():
        assert np.array_equal(got[k]["o_lat"], v["o_lat"])
    empty = np.full((wl.batch, 1, 50), -1, dtype=np.int32)
    got, err = O.sparse_decode_on_image(wl, qi, img["kv"], img["alpha_k"], inp["block_table"],
                                        inp["seq_lens"], empty, 3)
    assert not err
    for v in got.values():
        assert not np.any(v["o_lat"]) and np.isneginf(v["lse"])


# ---------------------------------------------------------------------------
# chunked prefill on the explicit path
# ---------------------------------------------------------------------------

def _prefill_images(wl, inp):
    img = O.full_cache_image(wl, inp)
    max_T = wl.max_pages_per_seq * wl.page_size
    e = O.expand_image(wl, img["kv"], img["alpha_k"], inp["block_table"], inp["seq_lens"],
                       inp["w_k"], inp["w_v"], inp["gamma_k"], max_T)
    return img, O.prefill_query_image(wl, inp), e


def check_expanded_keys_unit_rms():
    """Every materialised key divided by gamma_k has mean square
    m / (m + eps), m the mean square of its projection (the RMS of the
    stored latent's projection, through the stored alpha^k), and the rows
    past each sequence are zero."""
    wl = small("grouped")
    inp = W.make_inputs(wl, seed=37)
    img, _, e = _prefill_images(wl, inp)
    for b, T in enumerate(inp["seq_lens"]):
        T = int(T)
        t = np.arange(T)
        page, sl = inp["block_table"][b, t // 64], t % 64
        C = O.words_to_f64(img["kv"][page, sl, :wl.rank], wl.cache_dtype)
        for g in range(wl.groups):
            K = C @ inp["w_k"][g].astype(np.float64)
            m = np.mean(K * K, axis=1)
            got = np.mean((e["k_hat"][b, :T, g] / inp["gamma_k"][g][None, :]) ** 2, axis=1)
            assert np.allclose(got, m / (m + wl.eps), rtol=2e-6), np.max(np.abs(got / (m / (m + wl.eps)) - 1))
        assert not np.any(e["k_hat"][b, T:]) and not np.any(e["v"][b, T:])


def check_prefill_matches_explicit_f32():
    """With an fp32 cache the stored images differ from the inputs only by
    float32 rounding, so the prefill over them must agree with the explicit
    float64 path (values, latent-free) to ~1e-6; s_q > 1 exercises the causal
    window of every chunk token, G = 4 the per-group keys and values."""
    for name, kw in (("mtp", dict(s_q=6)), ("grouped", dict(s_q=3))):
        wl = small(name, **kw).replace(cache_dtype="f32")
        inp = W.make_inputs(wl, seed=38)
        img, qi, e = _prefill_images(wl, inp)
        res = O.prefill_on_images(wl, qi, e, img["kv"], inp["block_table"], inp["seq_lens"])
        for b in range(wl.batch):
            for i in range(wl.s_q):
                ex = O.explicit_rows(wl, inp, b, i)
                got = np.stack([res[(b, i, h)]["o"] for h in range(wl.heads)])
                lse = np.array([res[(b, i, h)]["lse"] for h in range(wl.heads)])
                assert rel_err(got, ex["o"]) < 2e-5, rel_err(got, ex["o"])
                assert np.max(np.abs(lse - ex["lse"])) < 2e-5


def check_prefill_bf16_within_tolerance():
    """The bf16 images alone (before any kernel) stay inside the 1e-2
    end-to-end budget against the explicit float64 path."""
    wl = small("dsv3", batch=1, seq_len=300, s_q=8)
    inp = W.make_inputs(wl, seed=39)
    img, qi, e = _prefill_images(wl, inp)
    res = O.prefill_on_images(wl, qi, e, img["kv"], inp["block_table"], inp["seq_lens"])
    worst = 0.0
    for i in range(wl.s_q):
        ex = O.explicit_rows(wl, inp, 0, i)
        got = np.stack([res[(0, i, h)]["o"] for h in range(wl.heads)])
        rowerr = np.max(np.abs(got - ex["o"]), axis=1) / np.max(np.abs(ex["o"]), axis=1)
        worst = max(worst, float(np.max(rowerr)))
    assert worst < 7.5e-3, worst
    return worst


# ---------------------------------------------------------------------------
# the GQA path of GQLA with QK-norm (per-group normed keys and values cached)
# ---------------------------------------------------------------------------

def check_gqa_image_against_torch():
    """Every row of the GQA-path cache against torch in float64: group g's key
    is torch's rms_norm of the stored latent's projection by W^K_g (weight
    gamma_k,g), its value the projection by W^V_g, at the offsets the layout
    states; the RoPE key words equal the latent cache's; slots never written
    keep the sentinel."""
    wl = small("grouped", batch=2, seq_len=90).replace(cache_dtype="f32")
    inp = W.make_inputs(wl, seed=41)
    gi = O.gqa_full_image(wl, inp)
    kvg = gi["kvg"]
    d, G = wl.head_dim, wl.groups
    assert kvg.shape[-1] == 2 * G * d + wl.rope_dim
    lat = O.full_cache_image(wl, inp)["kv"]
    written = np.zeros(kvg.shape[:2], dtype=bool)
    for b, T in enumerate(inp["seq_lens"]):
        T = int(T)
        o = inp["tok_offsets"]
        c = torch.from_numpy(np.asarray(inp["c"][o[b]:o[b + 1]], dtype=np.float32)).double()
        t = np.arange(T)
        page, sl = inp["block_table"][b, t // 64], t % 64
        written[page, sl] = True
        for g in range(G):
            k = torch.nn.functional.rms_norm(c @ torch.from_numpy(np.asarray(inp["w_k"][g], np.float64)),
                                             (d,), torch.from_numpy(np.asarray(inp["gamma_k"][g], np.float64)),
                                             wl.eps).numpy()
            v = (c @ torch.from_numpy(np.asarray(inp["w_v"][g], np.float64))).numpy()
            assert np.allclose(kvg[page, sl, 2 * d * g:2 * d * g + d], k, rtol=2e-7, atol=1e-30)
            assert np.allclose(kvg[page, sl, 2 * d * g + d:2 * d * (g + 1)], v, rtol=2e-7, atol=1e-6)
        assert np.array_equal(kvg[page, sl, 2 * d * G:], lat[page, sl, wl.rank:])
    assert np.all(np.isnan(kvg[~written]))


def _gqa_explicit_worst(wl, inp, num_splits):
    gi = O.gqa_full_image(wl, inp)
    qi = O.prefill_query_image(wl, inp)
    res = O.gqa_decode_on_image(wl, qi, gi["kvg"], inp["block_table"], inp["seq_lens"], num_splits)
    worst, worst_lse = 0.0, 0.0
    for b in range(wl.batch):
        for i in range(wl.s_q):
            ex = O.explicit_rows(wl, inp, b, i)
            got = np.stack([res[(b, i, h)]["o"] for h in range(wl.heads)])
            lse = np.array([res[(b, i, h)]["lse"] for h in range(wl.heads)])
            rowerr = np.max(np.abs(got - ex["o"]), axis=1) / np.max(np.abs(ex["o"]), axis=1)
            worst = max(worst, float(np.max(rowerr)))
            worst_lse = max(worst_lse, float(np.max(np.abs(lse - ex["lse"]))))
    return worst, worst_lse


def check_gqa_matches_explicit_f32():
    """With an fp32 cache the GQA-path decode over its stored cache equals the
    explicit float64 path to float32 rounding: s_q = 4 (every query's causal
    window, ragged lengths, shuffled pages) and G = 4 (per-group keys and
    values), 3 splits."""
    for name, kw in (("mtp", dict(s_q=4)), ("grouped", dict(s_q=3))):
        wl = small(name, **kw).replace(cache_dtype="f32")
        inp = W.make_inputs(wl, seed=42)
        worst, worst_lse = _gqa_explicit_worst(wl, inp, 3)
        assert worst < 2e-5 and worst_lse < 2e-5, (name, worst, worst_lse)


def check_gqa_equals_absorbed_f32():
    """The two algebraically equivalent paths of GQLA over the same weights:
    the GQA-path decode equals the absorbed decode followed by the value
    up-projection (float32 images of both caches)."""
    wl = small("grouped", s_q=2).replace(cache_dtype="f32")
    inp = W.make_inputs(wl, seed=43)
    gi = O.gqa_full_image(wl, inp)
    res = O.gqa_decode_on_image(wl, O.prefill_query_image(wl, inp), gi["kvg"], inp["block_table"],
                                inp["seq_lens"], 2)
    img = O.full_cache_image(wl, inp)
    ab = O.decode_on_image(wl, O.query_image(wl, inp), img["kv"], img["alpha_k"], inp["block_table"],
                           inp["seq_lens"], 2)
    for b in range(wl.batch):
        for i in range(wl.s_q):
            hs = list(range(wl.heads))
            o_ab = O.value_up_projection(wl, np.stack([ab[(b, i, h)]["o_lat"] for h in hs]),
                                         inp["w_v"], hs)
            o_gq = np.stack([res[(b, i, h)]["o"] for h in hs])
            assert rel_err(o_gq, o_ab) < 2e-5, rel_err(o_gq, o_ab)


def check_gqa_split_invariance():
    """Splitting the keys (whole pages) and merging the partials gives the
    unsplit result; a split past the visible tokens is empty (lse -inf)."""
    wl = small("mtp", s_q=4)
    inp = W.make_inputs(wl, seed=44)
    gi = O.gqa_full_image(wl, inp)
    qi = O.prefill_query_image(wl, inp)
    one = O.gqa_decode_on_image(wl, qi, gi["kvg"], inp["block_table"], inp["seq_lens"], 1)
    many = O.gqa_decode_on_image(wl, qi, gi["kvg"], inp["block_table"], inp["seq_lens"], 5)
    for key, v in one.items():
        assert rel_err(many[key]["o"], v["o"]) < 1e-12 and abs(many[key]["lse"] - v["lse"]) < 1e-12
        T = int(inp["seq_lens"][key[0]])
        for p, (lo, hi) in enumerate(O.split_bounds(T, 5)):
            if hi <= lo:
                assert many[key]["lse_part"][p] == -np.inf and not np.any(many[key]["o_part"][p])


def check_gqa_bf16_within_tolerance():
    """The bf16 GQA-path images alone (half keys and values, bf16 RoPE parts)
    stay inside the 1e-2 end-to-end budget against the explicit float64 path."""
    wl = small("dsv3", batch=2, seq_len=300, s_q=4)
    inp = W.make_inputs(wl, seed=45)
    worst, worst_lse = _gqa_explicit_worst(wl, inp, 2)
    assert worst < 7.5e-3 and worst_lse < 1e-2, (worst, worst_lse)
    return worst


def check_intensity_golden(golden):
    """The per-token arithmetic intensity of the absorbed decode path at s_q = 1,
    128 heads, r = 512, d_R = 64 against the value the GQLA page states."""
    wl = W.WORKLOADS["dsv3"]
    flops, nbytes = W.flops_and_bytes(wl.replace(groups=1), [1], cache_elem_bytes=2)
    nbytes_no_alpha = 2 * (wl.rank + wl.rope_dim)
    ai = flops / nbytes_no_alpha
    assert abs(ai - golden["value"]) <= golden["abs_tolerance"], ai
    return ai
