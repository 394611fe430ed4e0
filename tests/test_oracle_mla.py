"""Pins of the MLA (latent-cache) decode oracle against facts fixed outside it.

The pins: torch's scaled_dot_product_attention in float64 (a library routine)
on dense K = [c_kv, k_rope], V = c_kv; the decompression identity (multi-head
attention over K_h = [W_UK_h c, k_rope], V_h = W_UV_h c equals the absorbed
latent attention followed by W_UV_h), checked both with SDPA and with the
already-pinned paged MHA oracle; brute-force scatter through a random table;
closed forms and invariants. A planted mistake in the oracle must fail them.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
omla = sys.modules["oracle.mla_decode"]

D_C, D_R = 32, 8          # small latent and rope widths; the kernel's are 512 and 64


def scatter_latent(rows_list, pool_blocks, bs, x, rng):
    """Place per-sequence contiguous latent rows [L, W] into a random pool,
    one element at a time: pool[b, e // x, o, e % x] = row[t, e] with
    b = table[t // bs], o = t % bs."""
    width = rows_list[0].shape[1]
    pool = rng.standard_normal((pool_blocks, width // x, bs, x)).astype(np.float32)
    max_blocks = max(1, max(-(-r.shape[0] // bs) for r in rows_list))
    perm = rng.permutation(pool_blocks)
    table = np.zeros((len(rows_list), max_blocks), dtype=np.int32)
    pos = 0
    for s, rows in enumerate(rows_list):
        n = rows.shape[0]
        for i in range(-(-n // bs)):
            table[s, i] = perm[pos]
            pos += 1
        for t in range(n):
            b, o = table[s, t // bs], t % bs
            for e in range(width):
                pool[b, e // x, o, e % x] = rows[t, e]
    return pool, table


def problem(rng, lens, h, bs=16, x=4, extra=2):
    rows = [rng.standard_normal((n, D_C + D_R)).astype(np.float32) for n in lens]
    pool_blocks = sum(-(-n // bs) for n in lens) + extra
    pool, table = scatter_latent(rows, pool_blocks, bs, x, rng)
    q = rng.standard_normal((len(lens), h, D_C + D_R)).astype(np.float32)
    return q, rows, pool, table


def run(q, pool, table, lens, scale, latent_dim=D_C):
    return oracle.mla_decode(q, pool, table, np.asarray(lens, np.int32), scale, latent_dim,
                             q_kind="f32", kv_kind="f32")


def sdpa(q_sh, k, v, scale):
    """SDPA in float64: q [H, Dk], k [L, Dk], v [L, Dv] -> [H, Dv]."""
    h, dk = q_sh.shape
    qq = torch.from_numpy(np.asarray(q_sh, np.float64)).reshape(1, h, 1, dk)
    kk = torch.from_numpy(np.asarray(k, np.float64)).reshape(1, 1, -1, dk).expand(1, h, -1, dk)
    vv = torch.from_numpy(np.asarray(v, np.float64))
    vv = vv.reshape(1, 1, -1, vv.shape[-1]).expand(1, h, -1, vv.shape[-1])
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    return o.reshape(h, -1).numpy()


@pytest.mark.parametrize("bs", [16, 32])
def test_gather_latent_brute_force_and_x_invariance(bs):
    rng = np.random.default_rng(11)
    lens = [5, 33, 16, 70]
    rows = [rng.standard_normal((n, D_C + D_R)).astype(np.float32) for n in lens]
    for x in (1, 4, 8, D_C + D_R):
        pool, table = scatter_latent(rows, 12, bs, x, np.random.default_rng(x))
        for s, n in enumerate(lens):
            got = omla.gather_latent(pool, table[s], n)
            assert np.array_equal(got, rows[s])


@pytest.mark.parametrize("lens,h,bs", [([1, 17, 40], 4, 16), ([16, 32, 64], 16, 16), ([255, 3], 2, 16),
                                       ([1, 31, 32, 33, 100], 3, 32)])
def test_matches_dense_sdpa(lens, h, bs):
    rng = np.random.default_rng(len(lens) * 100 + h)
    q, rows, pool, table = problem(rng, lens, h, bs=bs)
    scale = 1.0 / np.sqrt(24.0)
    got = run(q, pool, table, lens, scale)
    for s, n in enumerate(lens):
        ref = sdpa(q[s], rows[s], rows[s][:, :D_C], scale)
        np.testing.assert_allclose(got[s], ref, rtol=1e-12, atol=1e-12)


def test_decompression_identity():
    """Absorbed latent attention, up-projected by W_UV_h, equals multi-head
    attention over K_h = [W_UK_h c, k_rope], V_h = W_UV_h c with query
    [q_nope_h, q_rope_h] when q_lat_h = [W_UK_h^T q_nope_h, q_rope_h]."""
    rng = np.random.default_rng(7)
    lens = [23, 48]
    h, d_nope, d_v = 4, 16, 12
    c = [rng.standard_normal((n, D_C)) for n in lens]
    kr = [rng.standard_normal((n, D_R)) for n in lens]
    w_uk = rng.standard_normal((h, d_nope, D_C)) / np.sqrt(D_C)
    w_uv = rng.standard_normal((h, d_v, D_C)) / np.sqrt(D_C)
    q_nope = rng.standard_normal((len(lens), h, d_nope))
    q_rope = rng.standard_normal((len(lens), h, D_R))
    scale = 1.0 / np.sqrt(d_nope + D_R)

    rows = [np.concatenate([c[s], kr[s]], axis=1).astype(np.float64) for s in range(len(lens))]
    pool, table = scatter_latent([r.astype(np.float32) for r in rows], 8, 16, 8, rng)
    # The latent rows went through float32: take the same rounding on both sides.
    rows32 = [r.astype(np.float32).astype(np.float64) for r in rows]
    q_lat = np.concatenate([np.einsum("hnc,shn->shc", w_uk, q_nope), q_rope], axis=2)
    latent_out = oracle.mla_decode(q_lat.astype(np.float32), pool, table,
                                   np.asarray(lens, np.int32), scale, D_C,
                                   q_kind="f32", kv_kind="f32")
    absorbed = np.einsum("hvc,shc->shv", w_uv, latent_out)

    # Multi-head attention over the decompressed K/V, per head, with the exact
    # (unabsorbed) query.
    for s, n in enumerate(lens):
        c32, r32 = rows32[s][:, :D_C], rows32[s][:, D_C:]
        ref = np.zeros((h, d_v))
        for hh in range(h):
            k_h = np.concatenate([c32 @ w_uk[hh].T, r32], axis=1)
            v_h = c32 @ w_uv[hh].T
            q_h = np.concatenate([q_nope[s, hh], q_rope[s, hh]])
            ref[hh] = sdpa(q_h[None, :], k_h, v_h, scale)[0]
        # q_lat was rounded to float32 before the oracle saw it: that moves the
        # logits by ~1e-7 relative, far below this tolerance and far above a
        # wrong formula.
        np.testing.assert_allclose(absorbed[s], ref, rtol=1e-5, atol=1e-6)

    # The same identity through the paged multi-head oracle (pinned on its
    # own): decompress into its K/V layouts, one kv head per query head.
    kp_list = []
    vp_list = []
    for s, n in enumerate(lens):
        c32, r32 = rows32[s][:, :D_C], rows32[s][:, D_C:]
        kh = np.stack([np.concatenate([c32 @ w_uk[hh].T, r32], axis=1) for hh in range(h)], axis=1)
        vh = np.stack([np.concatenate([c32 @ w_uv[hh].T, np.zeros((n, d_nope + D_R - d_v))], axis=1)
                       for hh in range(h)], axis=1)
        kp_list.append(kh)
        vp_list.append(vh)
    from tests.test_oracle_pins import scatter_to_pool
    kp, vp, tb = scatter_to_pool(kp_list, vp_list, 8, 16, 4, rng, dtype=np.float64)
    q_mha = np.concatenate([q_nope, q_rope], axis=2)
    mha = oracle.paged_decode(q_mha.astype(np.float32), kp.astype(np.float32), vp.astype(np.float32),
                              tb, np.asarray(lens, np.int32), scale, q_kind="f32", kv_kind="f32")
    # float32 rounding of the decompressed K/V and q is the only difference.
    np.testing.assert_allclose(absorbed, mha[:, :, :d_v], rtol=1e-4, atol=1e-5)


def test_physical_permutation_is_bitwise_invariant():
    rng = np.random.default_rng(3)
    lens = [40, 9]
    q, rows, pool, table = problem(rng, lens, 4, extra=5)
    base = run(q, pool, table, lens, 0.3)
    perm = rng.permutation(pool.shape[0])
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    pool2 = pool[perm]                       # new block j holds old block perm[j]
    table2 = inv[table].astype(np.int32)
    assert np.array_equal(run(q, pool2, table2, lens, 0.3), base)


def test_closed_forms():
    rng = np.random.default_rng(5)
    q, rows, pool, table = problem(rng, [1, 30], 3)
    out = run(q, pool, table, [1, 30], 0.7)
    # seq_len = 1: that token's c_kv row.
    np.testing.assert_array_equal(out[0], np.broadcast_to(rows[0][0, :D_C].astype(np.float64), (3, D_C)))
    # q = 0: uniform weights, the mean of the c_kv rows.
    qz = np.zeros_like(q)
    out0 = run(qz, pool, table, [1, 30], 0.7)
    np.testing.assert_allclose(out0[1], np.broadcast_to(rows[1][:, :D_C].astype(np.float64).mean(0), (3, D_C)),
                               rtol=1e-13, atol=1e-13)
    # seq_len = 0: zeros.
    assert not np.any(run(q, pool, table, [0, 0], 0.7))


def test_constant_latent_returns_the_constant():
    rng = np.random.default_rng(9)
    lens = [37]
    rows = [np.tile(rng.standard_normal((1, D_C + D_R)).astype(np.float32), (37, 1))]
    rows[0][:, D_C:] = rng.standard_normal((37, D_R))      # rope part varies: weights not uniform
    pool, table = scatter_latent(rows, 5, 16, 4, rng)
    q = rng.standard_normal((1, 4, D_C + D_R)).astype(np.float32)
    out = run(q, pool, table, lens, 0.5)
    np.testing.assert_allclose(out[0], np.broadcast_to(rows[0][0, :D_C].astype(np.float64), (4, D_C)),
                               rtol=1e-13, atol=1e-13)


def test_rope_only_logits():
    """With q's latent part zero, only k_rope decides the weights."""
    rng = np.random.default_rng(13)
    lens = [29]
    q, rows, pool, table = problem(rng, lens, 2)
    q[:, :, :D_C] = 0.0
    out = run(q, pool, table, lens, 0.4)
    r = rows[0].astype(np.float64)
    for hh in range(2):
        lg = 0.4 * (r[:, D_C:] @ q[0, hh, D_C:].astype(np.float64))
        w = np.exp(lg - lg.max())
        w /= w.sum()
        np.testing.assert_allclose(out[0, hh], w @ r[:, :D_C], rtol=1e-12, atol=1e-12)


def test_bf16_inputs_decode_exactly():
    rng = np.random.default_rng(17)
    lens = [20]
    q, rows, pool, table = problem(rng, lens, 2)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    pb = torch.from_numpy(pool).to(torch.bfloat16)
    got = oracle.mla_decode(qb.view(torch.int16).numpy().view(np.uint16),
                            pb.view(torch.int16).numpy().view(np.uint16), table,
                            np.asarray(lens, np.int32), 0.5, D_C, q_kind="bf16", kv_kind="bf16")
    ref = run(qb.float().numpy(), pb.float().numpy(), table, lens, 0.5)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# Planted mistakes must fail the pins above.
# ---------------------------------------------------------------------------

def _mutant_outputs(monkeypatch, fn):
    rng = np.random.default_rng(21)
    lens = [19, 40]
    q, rows, pool, table = problem(rng, lens, 4)
    ref = np.stack([sdpa(q[s], rows[s], rows[s][:, :D_C], 0.3) for s in range(2)])
    good = run(q, pool, table, lens, 0.3)
    np.testing.assert_allclose(good, ref, rtol=1e-12, atol=1e-12)
    fn(monkeypatch)
    bad = run(q, pool, table, lens, 0.3)
    return np.max(np.abs(bad - ref))


def test_pin_catches_value_from_the_wrong_slice(monkeypatch):
    def plant(mp):
        orig = omla.decode_cache_values

        def shifted(raw, kind, scale=1.0):   # rows shifted by the rope width
            v = orig(raw, kind, scale)
            return np.roll(v, -D_R, axis=-1) if v.ndim == 2 and v.shape[1] == D_C + D_R else v
        mp.setattr(omla, "decode_cache_values", shifted)
    assert _mutant_outputs(monkeypatch, plant) > 1e-3


def test_pin_catches_dropped_rope_term(monkeypatch):
    def plant(mp):
        orig = omla.gather_latent

        def no_rope(cache, row, n):
            r = orig(cache, row, n).copy()
            r[:, D_C:] = 0
            return r
        mp.setattr(omla, "gather_latent", no_rope)
    assert _mutant_outputs(monkeypatch, plant) > 1e-3


def test_pin_catches_swapped_slot_and_chunk(monkeypatch):
    def plant(mp):
        orig = omla.gather_latent

        def swapped(cache, row, n):
            nb, dx, bs, x = cache.shape
            bad = cache.reshape(nb, bs, dx, x).transpose(0, 2, 1, 3)
            return orig(np.ascontiguousarray(bad), row, n)
        mp.setattr(omla, "gather_latent", swapped)
    assert _mutant_outputs(monkeypatch, plant) > 1e-3


# --- appending latent rows ---------------------------------------------------

def _grown_problem(rng, lens, new, bs=16, x=4, extra=3):
    """Pool holding `lens` old rows per sequence (scattered element by element)
    with table room for `new` more tokens; returns the old rows, pool, table
    (blocks for the new tokens drawn from the free part of the pool) and new
    rows [S, new, W]."""
    width = D_C + D_R
    old = [rng.standard_normal((n, width)).astype(np.float32) for n in lens]
    need = [-(-(n + new) // bs) for n in lens]
    pool_blocks = sum(need) + extra
    pool = rng.standard_normal((pool_blocks, width // x, bs, x)).astype(np.float32)
    perm = rng.permutation(pool_blocks)
    table = np.full((len(lens), max(need)), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(lens):
        for i in range(need[s]):
            table[s, i] = perm[pos]
            pos += 1
        for t in range(n):
            b, o = table[s, t // bs], t % bs
            for e in range(width):
                pool[b, e // x, o, e % x] = old[s][t, e]
    rows = rng.standard_normal((len(lens), new, width)).astype(np.float32)
    return old, pool, table, rows


@pytest.mark.parametrize("x,bs", [(4, 16), (8, 16), (8, 32)])
def test_append_latent_read_back_through_the_gather(x, bs):
    rng = np.random.default_rng(41)
    lens, new = [0, 5, 16, 31, 33], 19
    old, pool, table, rows = _grown_problem(rng, lens, new, bs=bs, x=x)
    grown = oracle.append_latent(pool, rows, table, np.asarray(lens, np.int32))
    for s, n in enumerate(lens):
        got = oracle.gather_latent(grown, table[s], n + new)
        np.testing.assert_array_equal(got[:n], old[s])
        np.testing.assert_array_equal(got[n:], rows[s])


def test_append_latent_leaves_other_slots_bitwise_unchanged():
    rng = np.random.default_rng(42)
    lens, new, bs = [3, 17], 6, 16
    _, pool, table, rows = _grown_problem(rng, lens, new)
    grown = oracle.append_latent(pool, rows, table, np.asarray(lens, np.int32))
    named = set()
    for s, n in enumerate(lens):
        for p in range(n, n + new):
            named.add((int(table[s, p // bs]), p % bs))
    for b in range(pool.shape[0]):
        for o in range(bs):
            if (b, o) not in named:
                np.testing.assert_array_equal(grown[b, :, o, :], pool[b, :, o, :])


@pytest.mark.parametrize("bs", [16, 32])
def test_append_latent_brute_force_element_scatter(bs):
    rng = np.random.default_rng(43)
    lens, new, x = [7, 30, 62], 4, 4
    _, pool, table, rows = _grown_problem(rng, lens, new, bs=bs, x=x)
    want = pool.copy()
    for s, p0 in enumerate(lens):
        for j in range(new):
            p = p0 + j
            b, o = table[s, p // bs], p % bs
            for e in range(rows.shape[2]):
                want[b, e // x, o, e % x] = rows[s, j, e]
    got = oracle.append_latent(pool, rows, table, np.asarray(lens, np.int32))
    np.testing.assert_array_equal(got, want)


def test_append_latent_skip_rules():
    rng = np.random.default_rng(44)
    lens, new, bs = [10, 20, 5], 8, 16
    _, pool, table, rows = _grown_problem(rng, lens, new)
    table = table.copy()
    table[1, 1] = pool.shape[0]            # entry outside the pool: positions 20..27 go nowhere
    table[2, 1] = next(b for b in range(pool.shape[0]) if b not in table)   # room for 28..31
    positions = np.array([-1, 20, 28], np.int32)   # sequence 0 skipped; sequence 2 runs past its table
    grown = oracle.append_latent(pool, rows, table, positions)
    changed = np.argwhere(np.any(grown != pool, axis=(1, 3)))
    slots = {(int(b), int(o)) for b, o in changed}
    max_pos = table.shape[1] * bs
    assert max_pos == 32
    want = {(int(table[2, p // bs]), p % bs) for p in range(28, max_pos)}
    assert slots == want


def test_decode_after_append_matches_dense_attention():
    rng = np.random.default_rng(45)
    lens, new, h = [9, 33], 1, 3
    old, pool, table, rows = _grown_problem(rng, lens, new)
    grown = oracle.append_latent(pool, rows, table, np.asarray(lens, np.int32))
    new_lens = [n + new for n in lens]
    q = rng.standard_normal((len(lens), h, D_C + D_R)).astype(np.float32)
    got = run(q, grown, table, new_lens, 0.25)
    for s in range(len(lens)):
        full = np.concatenate([old[s], rows[s]])
        np.testing.assert_allclose(got[s], sdpa(q[s], full, full[:, :D_C], 0.25), rtol=1e-12, atol=1e-12)


def test_append_pins_catch_swapped_chunk_and_slot(monkeypatch):
    rng = np.random.default_rng(46)
    lens, new = [4, 18], 5
    old, pool, table, rows = _grown_problem(rng, lens, new)
    orig = omla.append_latent

    def swapped(cache, r, tab, pos):   # writes [b, o, c, i] instead of [b, c, o, i]
        nb, dx, bs, x = cache.shape
        view = np.ascontiguousarray(cache.reshape(nb, bs, dx, x).transpose(0, 2, 1, 3))
        out = orig(view, r, tab, pos)
        return np.ascontiguousarray(out.transpose(0, 2, 1, 3)).reshape(cache.shape)
    monkeypatch.setattr(oracle, "append_latent", swapped)
    grown = oracle.append_latent(pool, rows, table, np.asarray(lens, np.int32))
    got = oracle.gather_latent(grown, table[1], lens[1] + new)
    assert not np.array_equal(got[lens[1]:], rows[1])


# --- fp8 (e4m3fn) latent cache ---------------------------------------------

def _fp8_problem(rng, lens, h, d_c=32, d_r=16, bs=16, x=16):
    """Random e4m3fn code rows (NaN codes excluded) per sequence, scattered
    element by element into a pool of codes through a random table."""
    width = d_c + d_r
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    rows = [finite[rng.integers(0, finite.size, (n, width))] for n in lens]
    pool_blocks = sum(-(-n // bs) for n in lens) + 2
    pool = finite[rng.integers(0, finite.size, (pool_blocks, width // x, bs, x))]
    perm = rng.permutation(pool_blocks)
    table = np.zeros((len(lens), max(1, max(-(-n // bs) for n in lens))), np.int32)
    pos = 0
    for s, n in enumerate(lens):
        for i in range(-(-n // bs)):
            table[s, i] = perm[pos]
            pos += 1
        for t in range(n):
            for e in range(width):
                pool[table[s, t // bs], e // x, t % bs, e % x] = rows[s][t, e]
    q = rng.standard_normal((len(lens), h, width)).astype(np.float32)
    return q, rows, pool, table


def _torch_e4m3(codes, scale):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale


@pytest.mark.parametrize("kv_scale", [1.0, 0.0123, 3.5])
def test_fp8_cache_matches_sdpa_on_library_decoded_rows(kv_scale):
    rng = np.random.default_rng(51)
    lens, h, d_c = [1, 17, 40], 3, 32
    q, rows, pool, table = _fp8_problem(rng, lens, h, d_c=d_c)
    got = oracle.mla_decode(q, pool, table, np.asarray(lens, np.int32), 0.05, d_c, q_kind="f32",
                            kv_kind="e4m3fn", kv_scale=kv_scale)
    for s in range(len(lens)):
        full = _torch_e4m3(rows[s], kv_scale)
        np.testing.assert_allclose(got[s], sdpa(q[s], full, full[:, :d_c], 0.05), rtol=1e-12, atol=1e-12)


def test_fp8_pin_catches_dropped_scale(monkeypatch):
    rng = np.random.default_rng(52)
    lens, h, d_c = [9, 30], 2, 32
    q, rows, pool, table = _fp8_problem(rng, lens, h, d_c=d_c)
    orig = omla.decode_cache_values
    monkeypatch.setattr(omla, "decode_cache_values", lambda raw, kind, scale=1.0: orig(raw, kind))
    bad = oracle.mla_decode(q, pool, table, np.asarray(lens, np.int32), 0.05, d_c, q_kind="f32",
                            kv_kind="e4m3fn", kv_scale=0.25)
    full = _torch_e4m3(rows[1], 0.25)
    assert np.max(np.abs(bad[1] - sdpa(q[1], full, full[:, :d_c], 0.05))) > 1e-3


@pytest.mark.parametrize("kv_scale", [1.0, 0.02, 7.0])
def test_fp8_append_codes_match_library_conversion(kv_scale):
    """Codes read back through the gather equal torch's float8_e4m3fn
    conversion of the clamped float32 quotient; other slots unchanged."""
    rng = np.random.default_rng(53)
    lens, new, bs, x, width = [3, 16, 29], 5, 16, 16, 48
    pool_blocks = sum(-(-(n + new) // bs) for n in lens) + 2
    pool = rng.integers(0, 256, (pool_blocks, width // x, bs, x)).astype(np.uint8)
    perm = rng.permutation(pool_blocks)
    need = [-(-(n + new) // bs) for n in lens]
    table = np.full((len(lens), max(need)), -1, np.int32)
    pos = 0
    for s in range(len(lens)):
        for i in range(need[s]):
            table[s, i] = perm[pos]
            pos += 1
    vals = (rng.standard_normal((len(lens), new, width)) * 4).astype(np.float32)
    vals[0, 0, :4] = [1e6, -1e6, 0.0, -0.0]          # saturation and signed zeros
    bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    grown = oracle.append_latent(pool, bits, table, np.asarray(lens, np.int32), kv_kind="e4m3fn",
                                 kv_scale=kv_scale)
    f32 = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    quot = (f32 / torch.tensor(kv_scale, dtype=torch.float32)).clamp(-448.0, 448.0)
    want = quot.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for s, n in enumerate(lens):
        got = oracle.gather_latent(grown, table[s], n + new)
        np.testing.assert_array_equal(got[n:], want[s])
        np.testing.assert_array_equal(got[:n], oracle.gather_latent(pool, table[s], n))
