"""Pins of the oracle's main-attention prepare (normalised, rotated Q and the K/V cache write)
against closed forms, brute force, invariants and an independent fp8 conversion (torch).
CPU only."""

import numpy as np
import torch

from oracle import qsa as oq
from oracle.numerics import bf16_bits_to_f64, e4m3_bits_to_f64, f64_to_bf16_bits, round_bf16
from sparse_attention_qsa_amd.workloads import rotary_table

RNG = np.random.default_rng(777)
D = 128
NAN_BF16 = np.uint16(0x7FC0)


def _qkv(T, Hq, Hkv, q_heads, k_heads, v_heads):
    """main_qkv bits [T, (2Hq + 2Hkv)*128]: per Q head its q then a NaN-poisoned gate."""
    row = np.empty((T, (2 * Hq + 2 * Hkv) * D), np.uint16)
    qg = row[:, :2 * Hq * D].reshape(T, Hq, 2, D)
    qg[:, :, 0] = f64_to_bf16_bits(q_heads)
    qg[:, :, 1] = NAN_BF16
    row[:, 2 * Hq * D:(2 * Hq + Hkv) * D] = f64_to_bf16_bits(k_heads).reshape(T, Hkv * D)
    row[:, (2 * Hq + Hkv) * D:] = f64_to_bf16_bits(v_heads).reshape(T, Hkv * D)
    return row


def _bf16_ulps(a, b):
    return np.abs(f64_to_bf16_bits(a).astype(np.int64) - f64_to_bf16_bits(b).astype(np.int64))


def test_constant_vectors_closed_form_gate_never_read():
    """q = a*1 and k = b*1 at position 0 (rotation = identity): every output dim is
    (1 + w) * a / sqrt(a^2 + eps) up to the bf16 roundings of the chain; q uses the q weight,
    k the k weight; NaN gates never leak into Q or the cache."""
    T, Hq, Hkv, P = 3, 4, 2, 16
    eps = 1e-6
    a = round_bf16(RNG.uniform(0.5, 3.0, size=(T, Hq)))
    b = round_bf16(RNG.uniform(0.5, 3.0, size=(T, Hkv)))
    qh = np.repeat(a[:, :, None], D, axis=2)
    kh = np.repeat(b[:, :, None], D, axis=2)
    vh = round_bf16(RNG.standard_normal((T, Hkv, D)))
    qkv = _qkv(T, Hq, Hkv, qh, kh, vh)
    wq = f64_to_bf16_bits(round_bf16(RNG.normal(0, 0.1, D)))
    wk = f64_to_bf16_bits(round_bf16(RNG.normal(0, 0.1, D)))
    cache = np.zeros((4, Hkv, P, 2 * D), np.uint16)
    slots = np.array([5, 16 + 3, 3 * 16 + 15], np.int64)
    q, out = oq.prepare_main(qkv, np.zeros(T, np.int64), rotary_table(64), None, wq, wk, eps,
                             Hq, Hkv, cache, slots)
    qv = bf16_bits_to_f64(q)
    assert np.all(np.isfinite(qv))
    exp_q = (1.0 + bf16_bits_to_f64(wq))[None, None, :] * (a / np.sqrt(a * a + eps))[:, :, None]
    assert _bf16_ulps(qv, exp_q).max() <= 1
    for t, s in enumerate(slots):
        row = out[s // P, :, s % P]
        kv = bf16_bits_to_f64(row[:, :D])
        exp_k = (1.0 + bf16_bits_to_f64(wk))[None, :] * (b[t] / np.sqrt(b[t] ** 2 + eps))[:, None]
        assert _bf16_ulps(kv, exp_k).max() <= 1
        assert np.array_equal(row[:, D:], f64_to_bf16_bits(vh[t]))


def test_cache_scatter_brute_force_and_negative_slots_skipped():
    T, Hq, Hkv, P, pages = 40, 2, 2, 16, 8
    qkv = _qkv(T, Hq, Hkv, round_bf16(RNG.standard_normal((T, Hq, D))),
               round_bf16(RNG.standard_normal((T, Hkv, D))),
               round_bf16(RNG.standard_normal((T, Hkv, D))))
    cache = RNG.integers(0, 2 ** 16, size=(pages, Hkv, P, 2 * D)).astype(np.uint16)
    slots = RNG.permutation(pages * P)[:T].astype(np.int64)
    slots[::7] = -1
    w = f64_to_bf16_bits(np.zeros(D))
    q, out = oq.prepare_main(qkv, RNG.integers(0, 1000, T), rotary_table(2048), None, w, w,
                             1e-6, Hq, Hkv, cache, slots)
    written = np.zeros((pages, P), bool)
    v_bits = qkv[:, (2 * Hq + Hkv) * D:].reshape(T, Hkv, D)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        written[s // P, s % P] = True
        assert np.array_equal(out[s // P, :, s % P, D:], v_bits[t])
    # Every other row is untouched.
    assert np.array_equal(out.transpose(0, 2, 1, 3)[~written],
                          cache.transpose(0, 2, 1, 3)[~written])
    assert written.sum() == np.sum(slots >= 0)


def test_rotation_keeps_pass_through_dims_and_pair_norms():
    """The same rows at position 0 and at position p: dims 64..127 identical; each pair
    (i, i + 32), i < 32, keeps its length up to bf16 rounding."""
    T, Hq, Hkv = 16, 4, 1
    qh = round_bf16(RNG.standard_normal((T, Hq, D)))
    kh = round_bf16(RNG.standard_normal((T, Hkv, D)))
    qkv = _qkv(T, Hq, Hkv, qh, kh, kh)
    w = f64_to_bf16_bits(round_bf16(RNG.normal(0, 0.1, D)))
    table = rotary_table(4096)
    cache = np.zeros((T, Hkv, 1, 2 * D), np.uint16)
    slots = np.arange(T, dtype=np.int64)
    q0, c0 = oq.prepare_main(qkv, np.zeros(T, np.int64), table, None, w, w, 1e-6, Hq, Hkv,
                             cache, slots)
    pos = RNG.integers(1, 4096, T)
    q1, c1 = oq.prepare_main(qkv, pos, table, None, w, w, 1e-6, Hq, Hkv, cache, slots)
    for a, b in ((bf16_bits_to_f64(q0), bf16_bits_to_f64(q1)),
                 (bf16_bits_to_f64(c0[:, :, 0, :D]), bf16_bits_to_f64(c1[:, :, 0, :D]))):
        assert np.array_equal(a[..., 64:], b[..., 64:])
        n0 = np.hypot(a[..., :32], a[..., 32:64])
        n1 = np.hypot(b[..., :32], b[..., 32:64])
        assert np.all(np.abs(n1 - n0) <= 2.0 ** -7 * n0 + 1e-30)
    # And the rotation really acts (positions differ from zero).
    assert not np.array_equal(q0, q1)


def test_inner_product_of_rotated_q_and_k_depends_on_relative_position():
    """<q(m), k(n)> equals <q(m + d), k(n + d)> up to the bf16 roundings (NeoX rotation by a
    position-linear angle, as for the indexer)."""
    Hq, Hkv = 1, 1
    x = round_bf16(RNG.standard_normal((1, Hq, D)))
    y = round_bf16(RNG.standard_normal((1, Hkv, D)))
    w = f64_to_bf16_bits(np.zeros(D))
    table = rotary_table(8192)

    def qk(m, n):
        qkv = _qkv(1, Hq, Hkv, x, y, y)
        cache = np.zeros((1, 1, 1, 2 * D), np.uint16)
        q, _ = oq.prepare_main(qkv, np.array([m]), table, None, w, w, 1e-6, Hq, Hkv, cache,
                               np.array([-1]))
        _, c = oq.prepare_main(qkv, np.array([n]), table, None, w, w, 1e-6, Hq, Hkv, cache,
                               np.array([0]))
        return bf16_bits_to_f64(q[0, 0]) @ bf16_bits_to_f64(c[0, 0, 0, :D])

    base = qk(100, 37)
    for d in (1, 250, 3000):
        assert abs(qk(100 + d, 37 + d) - base) <= 0.05 * (1.0 + abs(base))


def test_scaled_e4m3_matches_torch_float8_and_saturates():
    scale = 0.0173
    x = np.concatenate([RNG.standard_normal(4000) * 3.0,
                        np.array([0.0, -0.0, 448 * scale, 447.9 * scale, 449 * scale,
                                  470 * scale, 1e4, -1e4, 2.0 ** -12, -(2.0 ** -9) * scale])])
    x = round_bf16(x)
    codes = oq.encode_scaled_e4m3(x, scale)
    q = (torch.tensor(x, dtype=torch.float64) / float(np.float32(scale))).to(torch.float32)
    ref = q.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.all((codes & 0x7F) != 0x7F)  # never a NaN code
    big = np.abs(x) >= 464 * scale
    assert np.all(np.abs(e4m3_bits_to_f64(codes[big])) == 448.0)


def test_fp8_cache_rows_are_the_scaled_values():
    T, Hq, Hkv, P = 6, 2, 2, 16
    kh = round_bf16(RNG.standard_normal((T, Hkv, D)))
    vh = round_bf16(RNG.standard_normal((T, Hkv, D)) * 4.0)
    qkv = _qkv(T, Hq, Hkv, round_bf16(RNG.standard_normal((T, Hq, D))), kh, vh)
    w = f64_to_bf16_bits(np.zeros(D))
    ks, vs = 0.02, 0.011
    cache = np.zeros((2, Hkv, P, 2 * D), np.uint8)
    slots = np.arange(T, dtype=np.int64) * 3
    _, out = oq.prepare_main(qkv, np.zeros(T, np.int64), rotary_table(64), None, w, w, 1e-6,
                             Hq, Hkv, cache, slots, kv_dtype="fp8", k_scale=ks, v_scale=vs)
    _, ref = oq.prepare_main(qkv, np.zeros(T, np.int64), rotary_table(64), None, w, w, 1e-6,
                             Hq, Hkv, np.zeros((2, Hkv, P, 2 * D), np.uint16), slots)
    for t, s in enumerate(slots):
        k_bf = bf16_bits_to_f64(ref[s // P, :, s % P, :D])
        v_bf = bf16_bits_to_f64(ref[s // P, :, s % P, D:])
        k8 = e4m3_bits_to_f64(out[s // P, :, s % P, :D]) * ks
        v8 = e4m3_bits_to_f64(out[s // P, :, s % P, D:]) * vs
        # e4m3: 3 mantissa bits (relative half-ulp 2^-4), subnormal step 2^-9 * scale.
        for got, want, sc in ((k8, k_bf, ks), (v8, v_bf, vs)):
            lim = np.minimum(np.abs(want), 448 * sc)
            err = np.abs(got - np.clip(want, -448 * sc, 448 * sc))
            assert np.all(err <= lim * 2.0 ** -4 + 2.0 ** -10 * sc + 1e-12)
