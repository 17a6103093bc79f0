"""Pins of the oracle's method steps against closed forms, independent libraries (torch
rms_norm / scaled_dot_product_attention in float64), exact integer arithmetic, brute force,
and invariants of the method.  CPU only."""

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import qsa as oq
from oracle.numerics import bf16_bits_to_f64, f64_to_bf16_bits, round_bf16
from sparse_attention_qsa_amd.workloads import make_workload, rotary_table
from tests.oracle_io import oracle_step, to_np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def rand_bf16(shape, std=1.0):
    return round_bf16(RNG.standard_normal(shape) * std)


def ulp_diff_bf16(a, b):
    ia = f64_to_bf16_bits(a).astype(np.int64)
    ib = f64_to_bf16_bits(b).astype(np.int64)
    return np.abs(ia - ib)


# ----------------------------------------------------------------------------- sums


def test_halving_sum_is_exact_on_integers_and_has_the_stated_order():
    x = RNG.integers(-1000, 1000, size=(50, 128)).astype(np.float64)
    assert np.array_equal(oq.halving_sum(x), x.sum(axis=1))


def test_halving_sum_order_pins_pairs_first_then_upper_half_onto_lower_half():
    """Values where the order decides the float64 result.  Each case is worked by hand from
    the stated order (adjacent pairs, then strides 32, 16, ..., 1); a sequential sum and a
    tree that keeps adding adjacent partials give a different answer on one of them."""
    # Case 1: dims 2 and 3 cancel inside their pair, so the 1 at dim 1 survives.
    #   halving: pair(0,1) = 1, pair(2,3) = 0 -> 1.   sequential: (1 + 2^60) - 2^60 = 0.
    v = np.zeros(128)
    v[1], v[2], v[3] = 1.0, 2.0 ** 60, -(2.0 ** 60)
    assert oq.halving_sum(v[None])[0] == 1.0
    assert np.cumsum(v)[-1] == 0.0                   # the order the pin rules out
    # Case 2: pair(0,1) = 2^60, pair(2,3) = 1, pair(64,65) = -2^60.  The stride-32 fold adds
    # pair 32 (dims 64, 65) onto pair 0 first -> 0, and pair 1 keeps its 1 -> 1.  A tree of
    # adjacent partials adds pair 1 onto pair 0 first and loses the 1 -> 0.
    v = np.zeros(128)
    v[0], v[2], v[64] = 2.0 ** 60, 1.0, -(2.0 ** 60)
    assert oq.halving_sum(v[None])[0] == 1.0
    t = v[0::2] + v[1::2]
    while len(t) > 1:
        t = t[0::2] + t[1::2]
    assert t[0] == 0.0                               # the adjacent tree the pin rules out
    # Case 3: the same with the big pair at stride 16 (pair 16 = dims 32, 33): the stride-32
    # fold leaves pair 16 alone and the stride-16 fold brings it onto pair 0.  2^60 + 1 at
    # pair 0 would swallow the 1 if pair 1 were added before pair 16.
    v = np.zeros(128)
    v[0], v[2], v[32] = 2.0 ** 60, 1.0, -(2.0 ** 60)
    assert oq.halving_sum(v[None])[0] == 1.0


# ----------------------------------------------------------------------------- RMSNorm


def test_rmsnorm_constant_vector_closed_form():
    w = rand_bf16(128, std=0.1)
    eps = 1e-6
    for a in [0.75, -3.0, 1.0 / 1024, 17.5]:
        x = np.full((1, 128), a)
        y = oq.gemma_rmsnorm(x, w, eps)[0]
        expect = a / np.sqrt(a * a + float(np.float32(eps))) * (1.0 + w)
        assert ulp_diff_bf16(y, expect).max() <= 1


def test_rmsnorm_zero_weight_gives_unit_rms():
    x = rand_bf16((64, 128))
    y = oq.gemma_rmsnorm(x, np.zeros(128), 1e-6)
    rms = np.sqrt((y * y).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 2 ** -7)


def test_rmsnorm_matches_torch_rms_norm_float64():
    x = rand_bf16((4000, 128))
    w = rand_bf16(128, std=0.1)
    eps = 1e-6
    ref = F.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(1.0 + w),
                     eps=float(np.float32(eps))).numpy()
    mine = oq.gemma_rmsnorm(x, w, eps)
    d = ulp_diff_bf16(mine, ref)
    assert d.max() <= 1            # only the last bit of a near-tie may differ
    assert (d == 0).mean() > 0.999


# ----------------------------------------------------------------------------- RoPE


def test_rotary_table_is_on_the_unit_circle():
    t = rotary_table(4096).numpy().astype(np.float64)
    assert np.abs(t[:, :32] ** 2 + t[:, 32:] ** 2 - 1).max() < 1e-6
    assert np.all(t[0, :32] == 1.0) and np.all(t[0, 32:] == 0.0)


def test_rope_position_zero_is_identity_and_pass_through_dims_untouched():
    tab = rotary_table(4096).numpy()
    y = rand_bf16((10, 128))
    cos, sin = oq.gather_cos_sin(tab, np.zeros(10, np.int64))
    assert np.array_equal(oq.neox_rope(y, cos, sin), y)
    cos, sin = oq.gather_cos_sin(tab, np.arange(10) * 97)
    assert np.array_equal(oq.neox_rope(y, cos, sin)[:, 64:], y[:, 64:])


def test_rope_is_a_rotation_of_pairs_i_and_i_plus_32():
    tab = rotary_table(8192).numpy()
    y = rand_bf16((200, 128))
    pos = RNG.integers(0, 8000, 200)
    cos, sin = oq.gather_cos_sin(tab, pos)
    z = oq.neox_rope(y, cos, sin)
    # Complex form: (a + i b) * e^{i theta}; norms of the pairs are preserved.
    a = y[:, :32] + 1j * y[:, 32:64]
    rot = a * (cos + 1j * sin)
    assert np.abs(z[:, :32] - rot.real).max() < 2 ** -7 * np.abs(rot.real).max()
    assert np.abs(z[:, 32:64] - rot.imag).max() < 2 ** -7 * np.abs(rot.imag).max()
    assert np.allclose(np.abs(a), np.abs(z[:, :32] + 1j * z[:, 32:64]), rtol=2 ** -7)


def test_rope_inner_product_depends_only_on_relative_position():
    tab = rotary_table(8192).numpy()
    q = rand_bf16((1, 128))
    k = rand_bf16((1, 128))

    def rot(v, p):
        c, s = oq.gather_cos_sin(tab, np.array([p]))
        return oq.neox_rope(v, c, s)[0]
    base = rot(q, 300) @ rot(k, 100)
    for m, n in [(1200, 1000), (5200, 5000), (200, 0)]:
        assert abs(rot(q, m) @ rot(k, n) - base) < 0.05 * (np.abs(q[0]) @ np.abs(k[0]))


def test_mrope_sections_and_equal_axes_reduce_to_1d():
    axis = oq.mrope_axis_of_pair((12, 10, 10))
    assert np.bincount(axis, minlength=3).tolist() == [12, 10, 10]
    tab = rotary_table(8192).numpy()
    y = rand_bf16((30, 128))
    p = RNG.integers(0, 8000, 30)
    c1, s1 = oq.gather_cos_sin(tab, p)
    c3, s3 = oq.gather_cos_sin(tab, np.stack([p, p, p], 1), (12, 10, 10))
    assert np.array_equal(oq.neox_rope(y, c1, s1), oq.neox_rope(y, c3, s3))
    # Moving only the H position changes exactly the H frequencies.
    trip = np.stack([p, p + 7, p], 1)
    c3, s3 = oq.gather_cos_sin(tab, trip, (12, 10, 10))
    changed = np.any(c3 != c1, axis=0)
    assert np.array_equal(changed, axis == 1)


# ----------------------------------------------------------------------------- compress


def _one_request_compress(raw, chunks, c, mrope=None, trip=None, ckv_pages=64):
    """Run compress_step over `raw` [L, 128] in the given chunks; returns the final state."""
    L = raw.shape[0]
    S, Pc = 16, 16
    tab = rotary_table(L + 256).numpy()
    w = f64_to_bf16_bits(rand_bf16(128, std=0.1)) if not hasattr(_one_request_compress, "w") \
        else _one_request_compress.w
    _one_request_compress.w = w
    state = oq.CompressState(ring=np.zeros((1, S, 128), np.uint16),
                             ring_pos=np.zeros((1, S, 3), np.int64) if mrope else None,
                             ckv=np.zeros((ckv_pages, Pc, 128), np.uint16))
    table = np.arange(ckv_pages, dtype=np.int32)[::-1].copy()[None, :]
    start = 0
    raw_bits = f64_to_bf16_bits(raw)
    for n in chunks:
        end = start + n
        pos = trip[start:end] if mrope else np.arange(start, end)
        state = oq.compress_step(np.array([0, n]), np.array([end]), raw_bits[start:end], pos,
                                 mrope, tab, w, 1e-6, np.array([0]), table, c, "bf16", state)
        start = end
    assert start == L
    return state


@pytest.mark.parametrize("c", [4, 8])
def test_compress_cache_bytes_do_not_depend_on_chunking(c):
    L = 203
    raw = rand_bf16((L, 128))
    whole = _one_request_compress(raw, [L], c)
    for chunks in ([1] * L, [5, 3, 1, 1, 7, 16, 2, 100, 68], [c - 1, 1, L - c]):
        part = _one_request_compress(raw, chunks, c)
        assert np.array_equal(part.ckv, whole.ckv)
        assert np.array_equal(part.ring, whole.ring)
    # The ring holds the last 16 raw keys in slots t % 16.
    bits = f64_to_bf16_bits(raw)
    for t in range(L - 16, L):
        assert np.array_equal(whole.ring[0, t % 16], bits[t])


def test_compress_mrope_chunking_invariance_uses_first_token_triples():
    L, c = 77, 8
    raw = rand_bf16((L, 128))
    t = np.arange(L)
    trip = np.stack([t, t + RNG.integers(0, 64, L), t + RNG.integers(0, 64, L)], 1)
    whole = _one_request_compress(raw, [L], c, (12, 10, 10), trip)
    part = _one_request_compress(raw, [3, 4, 4, 4, 4, 58], c, (12, 10, 10), trip)
    assert np.array_equal(part.ckv, whole.ckv)
    assert np.array_equal(part.ring_pos, whole.ring_pos)


def test_compress_of_identical_group_members_is_that_key_normalised_and_rotated():
    c, L = 4, 32
    keys = rand_bf16((L // c, 128))
    raw = np.repeat(keys, c, axis=0)
    st = _one_request_compress(raw, [L], c)
    w = bf16_bits_to_f64(_one_request_compress.w)
    tab = rotary_table(L + 256).numpy()
    cos, sin = oq.gather_cos_sin(tab, np.arange(0, L, c))
    expect = oq.neox_rope(oq.gemma_rmsnorm(keys, w, 1e-6), cos, sin)
    table = np.arange(64)[::-1]
    got = np.stack([bf16_bits_to_f64(st.ckv[table[g // 16], g % 16]) for g in range(L // c)])
    assert np.array_equal(got, expect)


def _groups_with_exact_distinct_means(n_groups, c, scale, rng):
    """Raw keys [n_groups * c, 128]: every member is an integer times `scale`, the members of
    a group are distinct and none is parallel to the group's mean, and each dim's sum is a
    multiple of c, so the mean is an integer times `scale` (exact in bf16)."""
    raw = np.empty((n_groups * c, 128))
    means = np.empty((n_groups, 128))
    for g in range(n_groups):
        members = rng.integers(-40, 41, size=(c - 1, 128))
        # The mean is the integer `target`; the last member makes the sum c * target.
        target = members.sum(axis=0) // c + rng.integers(-3, 4, size=128)
        last = c * target - members.sum(axis=0)
        grp = np.vstack([members, last[None, :]]).astype(np.float64)
        for m in grp:   # no member may point the same way as the mean
            assert abs(m @ target) < 0.999 * np.linalg.norm(m) * np.linalg.norm(target)
        raw[g * c:(g + 1) * c] = grp * scale
        means[g] = target * scale
    return raw, means


@pytest.mark.parametrize("c,chunks", [(4, [40]), (4, [9, 1, 13, 17]), (8, [40]),
                                      (8, [3, 30, 7])])
def test_compress_pools_the_mean_of_distinct_members(c, chunks):
    """[ops] qsa_compress_groups_with_ratio pools each completed group; the reading is the mean.
    With distinct integer members (scaled by 2^-14, so that RMSNorm's epsilon is not negligible)
    the expected row is written out here without compress_step: mean -> Gemma RMSNorm ->
    NeoX RoPE at the position of the group's first token.  Taking any one member, the sum, or
    another rotary position gives a different row."""
    rng = np.random.default_rng(2024 + c)
    L = 40
    raw, means = _groups_with_exact_distinct_means(L // c, c, 2.0 ** -14, rng)
    assert np.array_equal(round_bf16(raw), raw) and np.array_equal(round_bf16(means), means)
    st = _one_request_compress(raw, chunks, c)
    w = bf16_bits_to_f64(_one_request_compress.w)
    tab = rotary_table(L + 256).numpy().astype(np.float64)
    table = np.arange(64)[::-1]
    for g in range(L // c):
        m = means[g]
        # Gemma RMSNorm, written out: every square and the sum are exact here.
        inv = 1.0 / np.sqrt(np.sum(m * m) / 128.0 + float(np.float32(1e-6)))
        y = round_bf16((m * inv) * (1.0 + w))
        cos, sin = tab[g * c, :32], tab[g * c, 32:]
        a, b = y[:32], y[32:64]
        expect = y.copy()
        expect[:32] = round_bf16(a * cos - b * sin)
        expect[32:64] = round_bf16(b * cos + a * sin)
        got = bf16_bits_to_f64(st.ckv[table[g // 16], g % 16])
        assert np.array_equal(got, expect), g
        # The plausible wrong poolings differ from it.
        for wrong in (raw[g * c], raw[g * c + c - 1], c * m):
            inv_w = 1.0 / np.sqrt(np.sum(wrong * wrong) / 128.0 + float(np.float32(1e-6)))
            assert not np.array_equal(round_bf16((wrong * inv_w) * (1.0 + w)), y)


def _torch_norm_rope(x, w, pos_tab_rows):
    """bf16 rows x [..., 128] -> torch rms_norm (float64, weight 1 + w, the float32 epsilon)
    -> bf16 -> rotate-half RoPE of dims 0..63 with the given cos | sin rows -> bf16."""
    y = F.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(1.0 + w),
                   eps=float(np.float32(1e-6)))
    y = torch.from_numpy(round_bf16(y.numpy()))
    cs = torch.from_numpy(np.array(pos_tab_rows, dtype=np.float64))
    cos, sin = cs[..., :32], cs[..., 32:]
    a, b = y[..., :32], y[..., 32:64]
    out = y.clone()
    out[..., :32] = a * cos - b * sin
    out[..., 32:64] = b * cos + a * sin
    return round_bf16(out.numpy())


def test_prepare_index_q_normalises_then_rotates_every_head_at_the_row_position():
    """Indexer Q prep ([qsa] QSAIndexer.forward, unfused path): each head of a row through
    Gemma RMSNorm (here torch's rms_norm in float64), bf16, RoPE at the row's position, bf16.
    Only the last bit of a near-tie may differ from torch's summation order; skipping the
    norm, rotating at another position or mixing heads changes most values."""
    T, Hi = 8, 4
    x = rand_bf16((T, Hi, 128))
    w = rand_bf16(128, std=0.1)
    pos = RNG.integers(0, 900, size=T)
    tab = rotary_table(1024).numpy()
    codes, vals = oq.prepare_index_q(f64_to_bf16_bits(x.reshape(T, Hi * 128)), pos, tab, None,
                                     f64_to_bf16_bits(w), 1e-6, Hi, "bf16")
    rows = tab.astype(np.float64)[pos][:, None, :]               # [T, 1, 64]
    ref = _torch_norm_rope(x, w, np.broadcast_to(rows, (T, Hi, 64)))
    d = ulp_diff_bf16(vals, ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.995
    shifted = _torch_norm_rope(x, w, np.broadcast_to(tab.astype(np.float64)[pos + 1][:, None, :],
                                                     (T, Hi, 64)))
    assert (ulp_diff_bf16(vals, shifted) == 0).mean() < 0.9


def test_fp8_indexer_codes_are_the_bf16_prep_cast_to_e4m3():
    """With the e4m3 indexer the prepared bf16 Q is cast to e4m3fn ([qsa] QSAIndexer.forward:
    `.to(self.indexer_dtype)`): the codes equal torch's float8_e4m3fn cast of the bf16
    values, and decode back to those e4m3 values."""
    T, Hi = 8, 8
    x = rand_bf16((T, Hi * 128))
    w = f64_to_bf16_bits(rand_bf16(128, std=0.1))
    pos = RNG.integers(0, 900, size=T)
    tab = rotary_table(1024).numpy()
    _, v16 = oq.prepare_index_q(f64_to_bf16_bits(x), pos, tab, None, w, 1e-6, Hi, "bf16")
    c8, v8 = oq.prepare_index_q(f64_to_bf16_bits(x), pos, tab, None, w, 1e-6, Hi, "fp8")
    ref = torch.from_numpy(v16.astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(c8, ref.view(torch.uint8).numpy())
    assert np.array_equal(v8, ref.to(torch.float64).numpy())


def test_compress_rounds_the_pooled_mean_to_bf16_before_the_norm():
    """[ops] qsa_compress_groups_with_ratio returns the pooled row in bf16; the norm and the
    rotation then work on that row.  Random members make the mean rarely a bf16 value, so the
    rounding shows: the row matches mean -> bf16 -> norm -> RoPE (torch's rms_norm, as above)
    and not the chain that skips the first rounding."""
    c, L = 4, 128
    raw = rand_bf16((L, 128))
    st = _one_request_compress(raw, [L], c)
    w = bf16_bits_to_f64(_one_request_compress.w)
    tab = rotary_table(L + 256).numpy().astype(np.float64)
    mean = raw.reshape(L // c, c, 128).sum(axis=1) / c
    rows = tab[np.arange(0, L, c)]
    ref = _torch_norm_rope(round_bf16(mean), w, rows)
    unrounded = _torch_norm_rope(mean, w, rows)
    table = np.arange(64)[::-1]
    got = np.stack([bf16_bits_to_f64(st.ckv[table[g // 16], g % 16]) for g in range(L // c)])
    d = ulp_diff_bf16(got, ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.995
    assert (ulp_diff_bf16(got, unrounded) == 0).mean() < 0.95


# ----------------------------------------------------------------------------- scores / select


def test_scores_are_exact_on_small_integers():
    Hi, n = 4, 300
    q = RNG.integers(-8, 9, size=(Hi, 128)).astype(np.float64)
    k = RNG.integers(-8, 9, size=(n, 128)).astype(np.float64)
    exact = (k.astype(np.int64) @ q.astype(np.int64).T).sum(axis=1)
    assert np.array_equal(oq.index_scores(q, k), exact.astype(np.float64))


def test_scores_one_head_is_a_dot_product():
    q = rand_bf16((1, 128))
    k = rand_bf16((500, 128))
    assert np.allclose(oq.index_scores(q, k), k @ q[0], rtol=1e-13, atol=1e-12)


def test_select_matches_brute_force_sort_with_ties():
    for trial in range(20):
        n = int(RNG.integers(1, 400))
        kb = int(RNG.integers(1, 64))
        s = np.round(RNG.standard_normal(n), 1)      # many exact ties
        brute = sorted(range(n), key=lambda j: (-s[j], j))[:kb]
        assert np.array_equal(oq.select_blocks(s, kb), np.sort(brute))


def test_select_all_tied_takes_lowest_indices():
    assert np.array_equal(oq.select_blocks(np.zeros(100), 7), np.arange(7))


def _small_integer_index_case(idx_dtype, seed):
    """A batch for index_topk with small-integer queries and keys (every score is an exact
    integer, with many ties): 4 requests of 1, 3, 2 and 5 rows, compressed pages of 8 rows laid
    out by a seeded permutation, unused rows poisoned with NaN."""
    rng = np.random.default_rng(seed)
    c, budget, Pc, Hi = 4, 32, 8, 3
    lens = np.array([70, 37, 9, 130])
    nrows = np.array([1, 3, 2, 5])
    qsl = np.concatenate([[0], np.cumsum(nrows)])
    ncols = (lens // c + Pc - 1) // Pc
    pages = int(ncols.sum()) + 5
    perm = rng.permutation(pages)
    table = np.full((4, int(ncols.max())), -1, np.int64)
    k = 0
    for r in range(4):
        table[r, :ncols[r]] = perm[k:k + ncols[r]]
        k += ncols[r]
    key_int = rng.integers(-3, 4, size=(pages, Pc, 128))
    q_int = rng.integers(-3, 4, size=(int(qsl[-1]), Hi, 128))
    if idx_dtype == "bf16":
        enc = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(
            torch.int16).numpy().view(np.uint16)
        nan = np.uint16(0x7FC0)
    else:
        enc = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
        nan = np.uint8(0x7F)
    ckv = enc(key_int)
    used = np.zeros((pages, Pc), bool)
    for r in range(4):
        for j in range(lens[r] // c):
            used[table[r, j // Pc], j % Pc] = True
    ckv[~used] = nan
    return dict(c=c, budget=budget, lens=lens, qsl=qsl, table=table.astype(np.int32),
                key_int=key_int, q_int=q_int, ckv=ckv, q_codes=enc(q_int))


def _brute_force_packed(case):
    """Packed rows written out directly: dense keys gathered from the pages, integer scores,
    a full sort by (score descending, block ascending), then the blocks' tokens and the tail."""
    c, budget = case["c"], case["budget"]
    kb, W = budget // c, budget + c - 1
    qsl, lens = case["qsl"], case["lens"]
    out = np.full((int(qsl[-1]), W + 1), -1, np.int64)
    for r in range(len(lens)):
        n = qsl[r + 1] - qsl[r]
        for i in range(n):
            row = qsl[r] + i
            p = lens[r] - n + i
            vis = (p + 1) // c
            j = np.arange(vis)
            keys = case["key_int"][case["table"][r, j // 8], j % 8]          # [vis, 128]
            score = (keys.astype(np.int64) @ case["q_int"][row].T.astype(np.int64)).sum(1)
            order = sorted(range(vis), key=lambda b: (-score[b], b))
            chosen = sorted(order[:kb])
            toks = [t for b in chosen for t in range(b * c, b * c + c)]
            toks += list(range(vis * c, p + 1))
            out[row, :len(toks)] = toks
            out[row, W] = len(toks)
    return out


@pytest.mark.parametrize("idx_dtype,seed", [("bf16", 1), ("bf16", 2), ("fp8", 3)])
def test_index_topk_matches_brute_force_and_ignores_page_placement(idx_dtype, seed):
    """[qsa] QSAIndexer.forward: each row scores its own indexer Q against its request's
    compressed keys read through the compressed block table, keeps the budget / c best
    blocks and expands them.  Checked against a brute force written here (no oracle code),
    then the same batch with every compressed page moved and the table renumbered."""
    case = _small_integer_index_case(idx_dtype, seed)
    got = oq.index_topk(case["qsl"], case["lens"], case["q_codes"], case["ckv"],
                        case["table"], case["c"], case["budget"], idx_dtype)
    want = _brute_force_packed(case)
    assert np.array_equal(got, want)
    # Some rows really choose (vis > kb) and meet exact ties at the threshold.
    assert (got[:, -1] >= case["budget"]).sum() >= 6
    perm = np.random.default_rng(seed + 100).permutation(case["ckv"].shape[0])
    moved = np.empty_like(case["ckv"])
    moved[perm] = case["ckv"]
    table2 = np.where(case["table"] >= 0, perm[case["table"]], -1).astype(np.int32)
    again = oq.index_topk(case["qsl"], case["lens"], case["q_codes"], moved, table2, case["c"],
                          case["budget"], idx_dtype)
    assert np.array_equal(again, got)


# ----------------------------------------------------------------------------- expand


def test_compressed_keys_outside_the_cache_read_as_zero():
    """A visible block whose page is negative, past the cache, or past the block table's
    columns scores as an all-zero key (the oracle's reading; the GPU logits mask such keys
    the same way)."""
    ckv_vals = RNG.standard_normal((4, 16, 128)) + 5.0          # no zero anywhere
    row = np.array([2, 7, -1, 0], np.int32)                      # page 7 of 4 pages, then -1
    keys = oq.compressed_keys_of_request(ckv_vals, row, 64)
    assert np.array_equal(keys[:16], ckv_vals[2])
    assert np.all(keys[16:48] == 0.0)
    assert np.array_equal(keys[48:64], ckv_vals[0])
    short = oq.compressed_keys_of_request(ckv_vals, row[:2], 48)  # column 2 past the table
    assert np.array_equal(short[:16], ckv_vals[2])
    assert np.all(short[16:48] == 0.0)


def test_expand_closed_form_and_golden_tiny_decode_counts():
    with open(os.path.join(GOLDEN, "tiny_decode_counts.json")) as f:
        gold = json.load(f)
    c, budget = gold["compress_ratio"], gold["budget"]
    assert budget + c - 1 == gold["output_width"]
    for row in gold["rows"]:
        p = row["p"]
        vis = (p + 1) // c
        assert vis == row["visible_blocks"]
        blocks = np.arange(min(vis, budget // c)) * 3 % vis    # any kb distinct blocks
        blocks = np.unique(blocks)
        if len(blocks) < min(vis, budget // c):
            blocks = np.arange(min(vis, budget // c))
        packed = oq.expand_row(np.sort(blocks), p, c, budget)
        W = gold["output_width"]
        cnt = packed[W]
        assert cnt == row["count"]
        assert np.all(np.diff(packed[:cnt]) > 0) and packed[cnt - 1] <= p
        assert np.all(packed[cnt:W] == -1)
        assert np.array_equal(packed[cnt - row["tail"]:cnt], np.arange(vis * c, p + 1))


# ----------------------------------------------------------------------------- attention


def _dense_reference(q, K, V, scale):
    """torch SDPA (float64) of one row's heads over contiguous K/V [n, Hkv, D]."""
    Hq, Hkv = q.shape[0], K.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(q)[:, None, :]                      # [Hq, 1, D]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
    return F.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0, :].numpy()


def _tiny_attention_case(L=100, Hq=8, Hkv=2, P=16, seed=5):
    rng = np.random.default_rng(seed)
    pages_needed = (L + P - 1) // P
    pages = pages_needed + 3
    perm = rng.permutation(pages)[:pages_needed].astype(np.int32)
    kv = round_bf16(rng.standard_normal((pages, Hkv, P, 256)))
    bt = perm[None, :]
    q = round_bf16(rng.standard_normal((3, Hq, 128)))
    K = np.stack([kv[perm[t // P], :, t % P, :128] for t in range(L)])
    V = np.stack([kv[perm[t // P], :, t % P, 128:] for t in range(L)])
    return kv, bt, q, K, V


def test_sparse_gqa_dense_selection_matches_torch_sdpa():
    L, W = 100, 120
    kv, bt, q, K, V = _tiny_attention_case(L)
    ps = [99, 50, 0]
    packed = np.full((3, W + 1), -1, np.int32)
    for i, p in enumerate(ps):
        packed[i, :p + 1] = np.arange(p + 1)
        packed[i, W] = p + 1
    out = oq.sparse_gqa(f64_to_bf16_bits(q), f64_to_bf16_bits(kv), bt, np.zeros(3, np.int32),
                        packed)
    for i, p in enumerate(ps):
        ref = _dense_reference(q[i], K[:p + 1], V[:p + 1], 128 ** -0.5)
        assert np.abs(out[i] - ref).max() < 1e-12


def test_sparse_gqa_masks_invalid_entries_and_empty_rows():
    L, W = 100, 40
    kv, bt, q, K, V = _tiny_attention_case(L)
    sel = np.array([3, 17, 40, 41, 99])
    packed = np.full((4, W + 1), -1, np.int32)
    # row 0: the selection; row 1: same with -1 and out-of-table entries mixed in;
    # row 2: count 0.
    packed[0, :5] = sel
    packed[0, W] = 5
    packed[1, :9] = [3, -1, 17, 40, 5000, 41, -7, 99, -1]
    packed[1, W] = 9
    packed[2, W] = 0
    # row 3: row 0 with a count past W, which reads as W (the count column itself, 47 here,
    # would otherwise be taken for a token).
    packed[3] = packed[0]
    packed[3, W] = W + 7
    kvb = f64_to_bf16_bits(kv)
    out = oq.sparse_gqa(f64_to_bf16_bits(q[[0, 0, 0, 0]]), kvb, bt, np.zeros(4, np.int32),
                        packed)
    ref = _dense_reference(q[0], K[sel], V[sel], 128 ** -0.5)
    assert np.abs(out[0] - ref).max() < 1e-12
    assert np.abs(out[1] - ref).max() < 1e-12
    assert np.all(out[2] == 0.0)
    assert np.abs(out[3] - ref).max() < 1e-12


def test_sparse_gqa_gate_zero_halves_and_page_permutation_invariance():
    L, W = 100, 64
    kv, bt, q, K, V = _tiny_attention_case(L)
    packed = np.full((1, W + 1), -1, np.int32)
    packed[0, :10] = np.arange(0, 100, 10)
    packed[0, W] = 10
    kvb = f64_to_bf16_bits(kv)
    qb = f64_to_bf16_bits(q[:1])
    plain = oq.sparse_gqa(qb, kvb, bt, np.zeros(1, np.int32), packed)
    gated = oq.sparse_gqa(qb, kvb, bt, np.zeros(1, np.int32), packed,
                          gate=np.zeros((1, 8, 128), np.uint16))
    assert np.array_equal(gated, plain * 0.5)
    # Move every page elsewhere and renumber the table: same result.
    perm = np.random.default_rng(9).permutation(kv.shape[0])
    kv2 = np.empty_like(kvb)
    kv2[perm] = kvb
    out2 = oq.sparse_gqa(qb, kv2, perm[bt].astype(np.int32), np.zeros(1, np.int32), packed)
    assert np.array_equal(out2, plain)


def test_sparse_gqa_fp8_kv_matches_torch_sdpa_on_dequantized_values():
    """[fp8kv], e4m3 branch: K = code * k_scale, V = code * v_scale.  Pinned against torch's
    own float8_e4m3fn decoder and scaled_dot_product_attention (float64)."""
    L, W, Hq, Hkv, P = 100, 120, 8, 2, 16
    rng = np.random.default_rng(11)
    pages_needed = (L + P - 1) // P
    pages = pages_needed + 3
    perm = rng.permutation(pages)[:pages_needed].astype(np.int32)
    codes = rng.integers(0, 256, size=(pages, Hkv, P, 256)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes in the live cache
    k_scale, v_scale = 0.0317, 0.0453
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    K = np.stack([dec[perm[t // P], :, t % P, :128] for t in range(L)]) * k_scale
    V = np.stack([dec[perm[t // P], :, t % P, 128:] for t in range(L)]) * v_scale
    q = round_bf16(rng.standard_normal((2, Hq, 128)))
    packed = np.full((2, W + 1), -1, np.int32)
    packed[0, :L] = np.arange(L)
    packed[0, W] = L
    sel = np.array([2, 30, 31, 77])
    packed[1, :4] = sel
    packed[1, W] = 4
    out = oq.sparse_gqa(f64_to_bf16_bits(q), codes, perm[None, :], np.zeros(2, np.int32), packed,
                        kv_dtype="fp8", k_scale=k_scale, v_scale=v_scale)
    assert np.abs(out[0] - _dense_reference(q[0], K, V, 128 ** -0.5)).max() < 1e-12
    assert np.abs(out[1] - _dense_reference(q[1], K[sel], V[sel], 128 ** -0.5)).max() < 1e-12


# ----------------------------------------------------------------------------- end to end


def test_budget_at_least_context_reproduces_full_causal_attention():
    wl = make_workload("tiny_decode", budget=4096)
    st = oracle_step(wl)
    T = wl.num_tokens
    W = wl.output_width
    q = bf16_bits_to_f64(to_np(wl.q))
    kv = bf16_bits_to_f64(to_np(wl.kv_cache))
    bt = to_np(wl.block_table)[0]
    L = int(wl.seq_lens_host[0])
    K = np.stack([kv[bt[t // 16], :, t % 16, :128] for t in range(L)])
    V = np.stack([kv[bt[t // 16], :, t % 16, 128:] for t in range(L)])
    gate = bf16_bits_to_f64(to_np(wl.gate))
    for i in range(T):
        p = L - T + i
        assert st.packed[i, W] == p + 1
        assert np.array_equal(st.packed[i, :p + 1], np.arange(p + 1))
        ref = _dense_reference(q[i], K[:p + 1], V[:p + 1], 128 ** -0.5)
        ref = ref / (1.0 + np.exp(-gate[i]))
        assert np.abs(st.out[i] - ref).max() < 1e-12


def test_tiny_decode_selection_invariants_and_no_poison_read():
    wl = make_workload("tiny_decode")
    st = oracle_step(wl)
    W = wl.output_width
    L = int(wl.seq_lens_host[0])
    for i in range(wl.num_tokens):
        p = L - wl.num_tokens + i
        cnt = st.packed[i, W]
        row = st.packed[i, :cnt]
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] <= p
        tail = (p + 1) % wl.compress_ratio
        assert np.array_equal(row[cnt - tail:], np.arange(p + 1 - tail, p + 1))
        assert np.all(st.packed[i, cnt:W] == -1)
    assert np.all(np.isfinite(st.out))
    assert np.all(np.isfinite(bf16_bits_to_f64(st.q_codes)))


# ----------------------------------------------------------------------------- ReLU-sum switch


def test_relu_sum_scores_brute_force_and_special_cases():
    """agg "relu": sum over heads of max(0, q_h . k), against a plain float loop on small
    integers (exact); equal to the plain sum when every head's product is positive; 0 when
    every head's product is negative; never below the plain sum."""
    q = RNG.integers(-3, 4, size=(4, 128)).astype(np.float64)
    k = RNG.integers(-3, 4, size=(50, 128)).astype(np.float64)
    got = oq.index_scores(q, k, "relu")
    want = np.array([sum(max(0.0, float(np.dot(q[h], k[j]))) for h in range(4))
                     for j in range(50)])
    assert np.array_equal(got, want)
    assert np.all(got >= oq.index_scores(q, k))
    pos = np.abs(q)
    kp = np.abs(k) + 1.0
    assert np.array_equal(oq.index_scores(pos, kp, "relu"), oq.index_scores(pos, kp))
    assert np.all(oq.index_scores(pos, -kp, "relu") == 0.0)
    with pytest.raises(ValueError):
        oq.index_scores(q, k, "softmax")


def test_relu_sum_selection_differs_from_plain_sum_where_heads_disagree():
    """A block whose heads cancel (one strongly positive, one strongly negative) ranks low under
    the plain sum and high under ReLU-sum: the switch changes the selection."""
    q = np.zeros((2, 128))
    q[0, 0], q[1, 1] = 1.0, 1.0
    keys = np.zeros((4, 128))
    keys[0, 0], keys[0, 1] = 10.0, -10.0   # heads: +10, -10 -> sum 0, relu 10
    keys[1, 0], keys[1, 1] = 3.0, 0.0      # sum 3, relu 3
    keys[2, 0], keys[2, 1] = 2.0, 2.0      # sum 4, relu 4
    keys[3, 0], keys[3, 1] = -1.0, -1.0    # sum -2, relu 0
    assert list(oq.select_blocks(oq.index_scores(q, keys), 2)) == [1, 2]
    assert list(oq.select_blocks(oq.index_scores(q, keys, "relu"), 2)) == [0, 2]
