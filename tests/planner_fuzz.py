"""Random calls into the host side of a build of libmla_decode.so (no GPU).

    python tests/planner_fuzz.py LIB SEED CALLS

Drives the planner through its host-only entry points (single- and
multi-token previews) with random batches -- every cache format, page sizes
1..1024, empty and long sequences, split overrides, device sizes and a share
of malformed kv_indptr / kv_last_page_len / qo_indptr -- and the argument
checks of create / plan / run / destroy that come before any device call.
Meant for a sanitizer build (latent_attention_decode_amd.build with
sanitize=...): the sanitizer aborts the process on the first report.  Prints
one summary line.
"""

import ctypes
import sys

import numpy as np


def main(path: str, seed: int, calls: int) -> None:
    lib = ctypes.CDLL(path)
    I, P = ctypes.c_int, ctypes.c_void_p
    IP, SP = ctypes.POINTER(I), ctypes.POINTER(ctypes.c_size_t)
    lib.mla_decode_plan_preview.argtypes = [I, P, P, I, I, I, I, I, P, I, IP, IP, SP]
    lib.mla_decode_plan_preview_multi.argtypes = [I, P, P, P, I, I, I, I, I, P, I, IP, IP, SP]
    lib.mla_decode_create.argtypes = [ctypes.POINTER(P), I, I, I, I, ctypes.c_float, I, I]
    lib.mla_decode_plan.argtypes = [P, I, P, P, I, SP]
    lib.mla_decode_run.argtypes = [P, P, P, P, ctypes.c_int64, P, P, P, P, P, ctypes.c_size_t, P]
    lib.mla_decode_run_noalloc.argtypes = [P, P, P, P, ctypes.c_int64, P, P, P, P, P]
    lib.mla_decode_set_query_format.argtypes = [P, I]
    lib.mla_decode_destroy.argtypes = [P]
    lib.mla_decode_last_error.argtypes = [P]
    lib.mla_decode_last_error.restype = ctypes.c_char_p

    rng = np.random.default_rng(seed)
    accepted = items_total = 0
    for _ in range(calls):
        batch = int(rng.integers(1, 300))
        ps = int(rng.choice([1, 1, 2, 4, 16, 64, 1024]))
        lens = rng.integers(0, int(rng.choice([50, 3000, 20000])), size=batch)
        lens[rng.random(batch) < 0.1] = 0
        fmt = int(rng.integers(0, 3))
        pages = (lens + ps - 1) // ps
        indptr = np.concatenate([[int(rng.integers(0, 100))], pages]).cumsum().astype(np.int32)
        last = np.where(lens > 0, lens - ps * (pages - 1), int(rng.integers(1, ps + 1))).astype(np.int32)
        if rng.random() < 0.05:  # malformed: a decreasing kv_indptr, a last page too long
            if batch > 1:
                indptr[1], indptr[0] = indptr[0] + 5, indptr[1]
            if ps > 1:
                last[0] = ps + 1
        qo = None
        if rng.random() < 0.3:
            q = np.minimum(lens, rng.integers(0, 5, size=batch))
            if rng.random() < 0.05:
                q[0] = lens[0] + 1  # more query tokens than cache tokens
            qo = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
        split = int(rng.choice([0, 0, 0, 1, 3, 17, 300]))
        cus = int(rng.choice([1, 8, 80, 256, 304]))
        bpc = int(rng.choice([1, 2]))
        lp = last.ctypes.data if ps > 1 else None
        n, slots, ws = I(), I(), ctypes.c_size_t()

        def preview(buf, cap):
            if qo is None:
                return lib.mla_decode_plan_preview(batch, indptr.ctypes.data, lp, ps, fmt, split, cus, bpc, buf, cap,
                                                   ctypes.byref(n), ctypes.byref(slots), ctypes.byref(ws))
            return lib.mla_decode_plan_preview_multi(batch, qo.ctypes.data, indptr.ctypes.data, lp, ps, fmt, split,
                                                     cus, bpc, buf, cap, ctypes.byref(n), ctypes.byref(slots),
                                                     ctypes.byref(ws))

        preview(None, 0)
        if n.value > 0:
            items = np.zeros((n.value, 5), dtype=np.int32)
            if preview(items.ctypes.data, n.value) == 0:
                accepted += 1
                items_total += n.value
            # a buffer one item too small is refused without writing past it
            if n.value > 1:
                short = np.zeros((n.value, 5), dtype=np.int32)
                assert preview(short.ctypes.data, n.value - 1) != 0

    # Out-of-range enum values from a C caller.
    lib.mla_status_string.argtypes = [I]
    lib.mla_status_string.restype = ctypes.c_char_p
    assert lib.mla_status_string(42) and lib.mla_status_string(-1)
    ip = np.array([0, 100], dtype=np.int32)
    n, slots, ws0 = I(), I(), ctypes.c_size_t()
    assert lib.mla_decode_plan_preview(1, ip.ctypes.data, None, 1, 7, 0, 256, 1, None, 0, ctypes.byref(n),
                                       ctypes.byref(slots), ctypes.byref(ws0)) == 1

    # The handle's argument checks (nothing here reaches a device).
    h = P()
    assert lib.mla_decode_create(ctypes.byref(h), 0, 16, 576, 512, 1.0 / 24, 1, 2) == 0
    ws = ctypes.c_size_t()
    bad_indptr = np.array([0, 5, 3], dtype=np.int32)
    ones = np.ones(2, dtype=np.int32)
    assert lib.mla_decode_plan(h, 2, bad_indptr.ctypes.data, ones.ctypes.data, 0, ctypes.byref(ws)) == 1
    assert lib.mla_decode_plan(h, 0, bad_indptr.ctypes.data, ones.ctypes.data, 0, ctypes.byref(ws)) == 1
    assert lib.mla_decode_plan(h, 2, bad_indptr.ctypes.data, None, 0, ctypes.byref(ws)) == 1
    assert lib.mla_decode_run(h, 16, 16, 16, 0, 16, 16, 16, 16, None, 0, None) == 3
    assert lib.mla_decode_run_noalloc(h, 16, 16, 16, 0, 16, 16, 16, 16, None) == 3
    assert lib.mla_decode_last_error(h)
    for fmt_q, want in ((1, 0), (0, 0), (2, 1), (-5, 1)):
        assert lib.mla_decode_set_query_format(h, fmt_q) == want
    assert lib.mla_decode_set_query_format(None, 1) == 1
    assert lib.mla_decode_destroy(h) == 0
    assert lib.mla_decode_destroy(None) == 0
    for args in ((0, 8, 576, 512, 1.0, 1, 1), (0, 16, 576, 512, -1.0, 1, 1), (0, 16, 576, 512, 1.0, 1, 3),
                 (0, 16, 576, 512, 1.0, 7, 1)):
        h = P()
        assert lib.mla_decode_create(ctypes.byref(h), *args) != 0 and not h.value
    print(f"{calls} random plans, {accepted} accepted, {items_total} work items", flush=True)


if __name__ == "__main__":
    main(sys.argv[1], int(sys.argv[2]), int(sys.argv[3]))
