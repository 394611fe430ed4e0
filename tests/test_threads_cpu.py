"""The C ABI from several host threads at once, no GPU needed: every call
below fails host validation, so nothing is dereferenced or launched. Each
thread's pa_last_error() names its own failure (the text is thread-local),
however the threads interleave; ctypes releases the interpreter lock during
each foreign call, so the calls do run concurrently."""

import threading

from tests.test_abi_cpu import APPEND, pa  # noqa: F401  (module fixture)

A = 1 << 20


def test_last_error_is_per_thread(pa):  # noqa: F811
    n = 3000
    start = threading.Barrier(3)
    bad = []

    def mla():        # num_heads 0
        start.wait()
        for _ in range(n):
            rc = pa.pa_mla_decode(A, 2 * A, 3 * A, 4, 0, 64, 0.1, 4 * A, 8, 5 * A, 16, 128, 6 * A, 1 << 40, None)
            msg = pa.pa_last_error()
            if rc != pa.PA_ERR_SHAPE or "num_heads 0" not in msg:
                bad.append(("mla", rc, msg))

    def append():     # head_size 96
        start.wait()
        a = dict(APPEND, head_size=96)
        for _ in range(n):
            rc = pa.pa_kv_cache_append(*a.values())
            msg = pa.pa_last_error()
            if rc != pa.PA_ERR_SHAPE or "96" not in msg:
                bad.append(("append", rc, msg))

    def latent():     # misaligned rows
        start.wait()
        for _ in range(n):
            rc = pa.pa_mla_cache_append(A, 2 * A + 4, 4, 1, 64, 3 * A, 8, 4 * A, 16, None)
            msg = pa.pa_last_error()
            if rc != pa.PA_ERR_ALIGN or "aligned" not in msg:
                bad.append(("latent", rc, msg))

    threads = [threading.Thread(target=f) for f in (mla, append, latent)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:3]
