"""Host-side checks of the latent-cache (MLA) entry points, no GPU needed:
every call below fails validation or is the num_seqs == 0 no-op, so the fake
(aligned) device addresses are never dereferenced and nothing is launched."""

import pytest
import torch

from tests.test_abi_cpu import pa  # noqa: F401  (module fixture)

A = 1 << 20          # fake, 16-byte aligned device address


def call(pa, **over):
    args = dict(out=A, query=2 * A, latent=3 * A, S=4, H=16, nb=64, scale=0.1, table=4 * A, mb=8,
                lens=5 * A, bs=16, msl=128, ws=6 * A, wsb=1 << 40, stream=None)
    args.update(over)
    return pa.pa_mla_decode(args["out"], args["query"], args["latent"], args["S"], args["H"], args["nb"],
                            args["scale"], args["table"], args["mb"], args["lens"], args["bs"], args["msl"],
                            args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(H=0), -2), (dict(H=129), -2), (dict(S=-1), -2), (dict(S=65536), -2),
    (dict(bs=64), -2), (dict(msl=-1), -2), (dict(msl=129), -2), (dict(nb=0), -2), (dict(mb=0), -2),
    (dict(scale=float("nan")), -2), (dict(out=None), -1), (dict(query=None), -1), (dict(latent=None), -1),
    (dict(table=None), -1), (dict(lens=None), -1), (dict(out=A + 8), -5), (dict(latent=A + 4), -5),
    (dict(lens=5 * A + 2), -5), (dict(ws=None), -4), (dict(wsb=16), -4), (dict(ws=6 * A + 8), -5),
    (dict(out=2 * A + 64), -2),
])
def test_validation_rejects(pa, over, code):  # noqa: F811
    assert call(pa, **over) == code
    assert pa.pa_last_error()


def test_zero_sequences_is_a_noop(pa):  # noqa: F811
    assert call(pa, S=0, out=None, query=None, latent=None, table=None, lens=None, ws=None, wsb=0) == 0
    assert pa.pa_mla_workspace_bytes(0, 16) == 0


def test_workspace_grows_with_heads_and_sequences(pa):  # noqa: F811
    # one bf16 partial row per (slot, head), slots = sequences + stream-K
    # shares (at least 512 shares of one 16-head wave on 256 compute units)
    w16 = pa.pa_mla_workspace_bytes(256, 16)
    assert w16 >= (256 + 512) * 16 * 512 * 2
    assert pa.pa_mla_workspace_bytes(256, 17) > w16
    assert pa.pa_mla_workspace_bytes(512, 16) > w16
    with pytest.raises(ValueError):
        pa.pa_mla_workspace_bytes(4, 0)


def test_tensor_call_refuses_cpu_and_wrong_shapes(pa):  # noqa: F811
    q = torch.zeros(2, 16, 576, dtype=torch.bfloat16)
    out = torch.zeros(2, 16, 512, dtype=torch.bfloat16)
    cache = torch.zeros(pa.mla_cache_shape(4), dtype=torch.bfloat16)
    tbl = torch.zeros(2, 1, dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        pa.mla_decode(out, q, cache, 0.1, tbl, lens, 16)
    assert pa.mla_cache_shape(4) == (4, 72, 16, 8)


APPEND = dict(latent=A, rows=2 * A, S=4, T=1, nb=64, table=3 * A, mb=8, pos=4 * A, bs=16, stream=None)


def call_append(pa, **over):
    a = dict(APPEND)
    a.update(over)
    return pa.pa_mla_cache_append(a["latent"], a["rows"], a["S"], a["T"], a["nb"], a["table"], a["mb"],
                                  a["pos"], a["bs"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(S=-1), -2), (dict(T=0), -2), (dict(bs=64), -2), (dict(nb=0), -2), (dict(mb=0), -2),
    (dict(S=1 << 20, T=1 << 11), -2), (dict(latent=None), -1), (dict(rows=None), -1),
    (dict(table=None), -1), (dict(pos=None), -1), (dict(latent=A + 8), -5), (dict(rows=2 * A + 4), -5),
    (dict(table=3 * A + 2), -5), (dict(pos=4 * A + 1), -5),
    (dict(rows=A + 64 * 18432 - 16), -2),   # rows start inside the cache
    (dict(rows=A - 1152 * 4 + 16), -2),     # rows end inside the cache
])
def test_append_validation_rejects(pa, over, code):  # noqa: F811
    assert call_append(pa, **over) == code
    assert pa.pa_last_error()


def test_append_zero_sequences_is_a_noop(pa):  # noqa: F811
    assert call_append(pa, S=0, latent=None, rows=None, table=None, pos=None) == 0


def test_tensor_append_refuses_cpu_tensors(pa):  # noqa: F811
    cache = torch.zeros(pa.mla_cache_shape(4), dtype=torch.bfloat16)
    rows = torch.zeros(2, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        pa.mla_cache_append(cache, rows, torch.zeros(2, 1, dtype=torch.int32), torch.zeros(2, dtype=torch.int32))


def call_fp8(pa, **over):
    args = dict(out=A, query=2 * A, latent=3 * A, S=4, H=16, nb=64, scale=0.1, table=4 * A, mb=8,
                lens=5 * A, bs=16, msl=128, ks=7 * A, ws=6 * A, wsb=1 << 40, stream=None)
    args.update(over)
    return pa.pa_mla_decode_fp8(args["out"], args["query"], args["latent"], args["S"], args["H"], args["nb"],
                                args["scale"], args["table"], args["mb"], args["lens"], args["bs"], args["msl"],
                                args["ks"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(H=0), -2), (dict(H=129), -2), (dict(bs=64), -2), (dict(msl=129), -2), (dict(latent=None), -1),
    (dict(latent=A + 8), -5), (dict(ks=7 * A + 2), -5), (dict(ws=None), -4), (dict(out=2 * A + 64), -2),
])
def test_fp8_decode_validation_rejects(pa, over, code):  # noqa: F811
    assert call_fp8(pa, **over) == code
    assert pa.pa_last_error()


def test_fp8_decode_zero_sequences_is_a_noop(pa):  # noqa: F811
    assert call_fp8(pa, S=0, out=None, query=None, latent=None, table=None, lens=None, ws=None, wsb=0) == 0


def test_fp8_append_validation(pa):  # noqa: F811
    a = dict(APPEND)
    f = pa.pa_mla_cache_append_fp8
    args = [a["latent"], a["rows"], a["S"], a["T"], a["nb"], a["table"], a["mb"], a["pos"], a["bs"], 8 * A, None]
    bad = list(args)
    bad[9] = 8 * A + 2
    assert f(*bad) == -5
    bad = list(args)
    bad[8] = 64
    assert f(*bad) == -2
    bad = list(args)
    bad[1] = A + 64 * 9216 - 16          # rows start inside the (9 KiB-block) cache
    assert f(*bad) == -2
    bad = list(args)
    bad[1] = A + 64 * 9216               # just past it: accepted by the overlap check, rejected nowhere else
    bad[0] = None
    assert f(*bad) == -1
