"""Every real row of a full-size attention output against the fp64 oracle:
one query head per worker process (test infrastructure; numpy and the
oracle only, nothing here touches the GPU).

The parent writes the inputs, the lists and the GPU's output and lse to a
scratch directory; spawned workers (BLAS limited to one thread each) map
them, run ``oracle.attend`` for their head and return that head's error
statistics."""
import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

MAX_WORKERS = 16


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _head_errors(args):
    path, lay, h = args
    from threadpoolctl import threadpool_limits

    import oracle
    load = lambda n: np.load(os.path.join(path, n + ".npy"), mmap_mode="r")
    q, k, v, out, lse, idx, cnt = (load(n) for n in ("q", "k", "v", "out", "lse", "idx", "cnt"))
    g = h // (lay["num_q_heads"] // lay["num_kv_heads"])
    lay1 = dict(lay, num_q_heads=1, num_kv_heads=1)
    with threadpool_limits(1):
        ro, rl = oracle.attend(lay1, np.ascontiguousarray(q[:, :, h:h + 1]),
                               np.ascontiguousarray(k[:, :, g:g + 1]),
                               np.ascontiguousarray(v[:, :, g:g + 1]),
                               np.ascontiguousarray(idx[:, h:h + 1]),
                               np.ascontiguousarray(cnt[:, h:h + 1]))
    rows = np.arange(lay["q_len"]) < lay["q_valid"]
    got = _bf16_to_f64(out[:, :, h])                       # [B, q_len, D]
    err = np.abs(got[:, rows] - ro[:, rows, 0])
    gl = np.asarray(lse[:, h], dtype=np.float64)           # [B, q_len]
    rl = rl[:, 0]
    fin = np.isfinite(rl)
    lse_ok = bool(np.array_equal(np.isfinite(gl), fin))
    lse_err = float(np.abs(gl[fin] - rl[fin]).max()) if fin.any() else 0.0
    pad_zero = bool((got[:, ~rows] == 0).all())
    return h, float(err.max()) if err.size else 0.0, float(err.sum()), int(err.size), pad_zero, \
        lse_ok, lse_err


def check_every_row(case, idx, cnt, out_bits, lse):
    """case: the synthetic case (bf16 bits); idx, cnt: the lists the GPU ran;
    out_bits: the GPU output as uint16 bf16 bits [B, q_len, Hq, D]; lse: fp32
    [B, Hq, q_len]. Returns (max-abs, mean-abs over real rows, lse max-abs,
    padded rows all zero, lse finite where the oracle's is)."""
    lay = case.layout
    base = "/dev/shm" if os.path.isdir("/dev/shm") and os.access("/dev/shm", os.W_OK) else None
    need = sum(a.nbytes for a in (case.q, case.k, case.v, out_bits, lse, idx, cnt))
    if base is not None:
        st = os.statvfs(base)
        if st.f_bavail * st.f_frsize < 2 * need:
            base = None
    path = tempfile.mkdtemp(prefix="bsattn_full_", dir=base)
    try:
        for n, a in (("q", case.q), ("k", case.k), ("v", case.v), ("out", out_bits), ("lse", lse),
                     ("idx", idx), ("cnt", cnt)):
            np.save(os.path.join(path, n + ".npy"), np.ascontiguousarray(a))
        workers = max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0)), lay["num_q_heads"]))
        with mp.get_context("spawn").Pool(workers) as pool:
            res = pool.map(_head_errors, [(path, lay, h) for h in range(lay["num_q_heads"])],
                           chunksize=1)
    finally:
        shutil.rmtree(path, ignore_errors=True)
    mx = max(r[1] for r in res)
    mean = sum(r[2] for r in res) / max(1, sum(r[3] for r in res))
    return mx, mean, max(r[6] for r in res), all(r[4] for r in res), all(r[5] for r in res)
