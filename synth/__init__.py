"""Seeded synthetic inputs for selected-block attention.

This module is the single source of input bytes for both the fp64 CPU oracle
and the GPU library. It draws random numbers and lays them out; it computes
nothing of the method itself (no pooling, scoring, selection or softmax).

Layout of every case (all arrays are numpy ``uint16`` holding bf16 bit
patterns, C-contiguous):

* ``q``: ``[B, q_len, Hq, D]``. Query rows are the generation tokens; rows
  ``>= q_valid`` are padding.
* ``k``, ``v``: ``[B, kv_len, Hkv, D]``. Keys are ``cat(prefix, gen)``. The
  prefix segment ``[0, kv_prefix_len)`` holds ``kv_prefix_valid`` real keys
  followed by padding; the generation segment starts at ``kv_prefix_len`` and
  holds ``kv_suffix_valid`` real keys followed by padding. Each segment is
  padded on its own up to a block multiple, which is how the two-stream
  Cosmos 3 helper pads its understanding and generation pathways (diffusers
  ``cosmos_parallel.py``, ``shard_cosmos3_sequence``).

Values: fp64 draws, rounded to fp32 and then to bf16 (round to nearest even
at each step). Seeds are ``SeedSequence([42, cfg, layer, stream, ...])`` with
stream 0 = Q, 1 = K, 2 = V, 3 = structure, 4 = row sampling (Q/K/V rows add
batch row, segment and a 2048-row chunk number to the key); 42 is the
generation seed the Cosmos3-Nano and MiniMax H3 measurements used (vllm-omni
PR #8583 "Test Result"; PR #8644 "Test Plan").
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

SEED = 42
STREAM_Q, STREAM_K, STREAM_V, STREAM_STRUCT, STREAM_ROWS = 0, 1, 2, 3, 4

# Named workloads. ``frames`` is (latent frames, patch rows, patch cols) of the
# generation tokens, raster order, frame-major.
CONFIGS = {
    "tiny": dict(cfg=1, batch=1, hq=2, hkv=1, d=64, prefix=64, gen=448,
                 bq=64, bk=64, sparsity=50, dist="normal"),
    "dense8k": dict(cfg=2, batch=1, hq=32, hkv=8, d=128, prefix=0, gen=8192,
                    bq=128, bk=128, sparsity=0, dist="normal"),
    "edge48k": dict(cfg=3, batch=1, hq=32, hkv=8, d=128, prefix=512, gen=48360,
                    frames=(31, 30, 52), bq=64, bk=64, sparsity=75, dist="lowrank"),
    "video720p": dict(cfg=4, batch=1, hq=32, hkv=8, d=128, prefix=512, gen=172800,
                      frames=(48, 45, 80), bq=128, bk=128, sparsity=75, dist="lowrank"),
    # Other geometries and head layouts at the 48k edge-video token shape:
    # 256x128 blocks (the pages' Blackwell validation geometry), MHA at
    # head_dim 64, MQA.
    "edge48k_256x128": dict(cfg=6, batch=1, hq=32, hkv=8, d=128, prefix=512, gen=48360,
                            frames=(31, 30, 52), bq=256, bk=128, sparsity=75, dist="lowrank"),
    "mha64_48k": dict(cfg=7, batch=1, hq=32, hkv=32, d=64, prefix=512, gen=48360,
                      frames=(31, 30, 52), bq=64, bk=64, sparsity=75, dist="lowrank"),
    "mqa48k": dict(cfg=8, batch=1, hq=32, hkv=1, d=128, prefix=512, gen=48360,
                   frames=(31, 30, 52), bq=64, bk=64, sparsity=75, dist="lowrank"),
    # One GPU's share of the 48k workload split over eight GPUs by heads
    # (4 query heads and their KV head, the full sequence).
    "edge48k_cp8": dict(cfg=9, batch=1, hq=4, hkv=1, d=128, prefix=512, gen=48360,
                        frames=(31, 30, 52), bq=64, bk=64, sparsity=75, dist="lowrank"),
    # Two-stream schedule: 36 layers, layers < 8 dense, the rest 75 % sparse.
    "twostream": dict(cfg=5, batch=1, hq=32, hkv=8, d=128, prefix=1000, gen=20000,
                      bq=128, bk=128, sparsity=75, dist="normal",
                      layers=36, dense_layers=8),
}


def round_up(n: int, m: int) -> int:
    return ((n + m - 1) // m) * m


@dataclass
class Case:
    """One synthetic input set. ``layout`` is a plain dict of shape integers."""
    name: str
    layout: dict
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    sparsity: int
    meta: dict = field(default_factory=dict)


def make_layout(batch, hq, hkv, d, bq, bk, prefix, gen, scale=None):
    """Padded sizes of a case: each segment rounded up to its block size."""
    prefix_len = round_up(prefix, bk)
    q_len = round_up(gen, bq)
    gen_k_len = round_up(gen, bk)
    return dict(
        batch=batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_q=bq, block_k=bk,
        q_len=q_len, q_valid=gen,
        kv_prefix_len=prefix_len, kv_prefix_valid=prefix,
        kv_len=prefix_len + gen_k_len, kv_suffix_valid=gen,
        scale=(1.0 / math.sqrt(d)) if scale is None else float(scale),
    )


def rng_for(cfg: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, cfg, layer, stream])))


def to_bf16_bits(x) -> np.ndarray:
    """fp64/fp32 values -> bf16 bit patterns (fp64 -> fp32 -> bf16, each RNE)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


CHUNK_ROWS = 2048


def _chunk_rng(key, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, *key, chunk])))


def _gen_rows(key, rows, heads, d, add=None):
    """[rows, heads, d] bf16 bits of i.i.d. N(0,1) fp64 draws (+ ``add(t0, t1)``).

    Rows are drawn in chunks of CHUNK_ROWS; chunk c draws from its own
    generator seeded with ``SeedSequence([42, *key, c])``, so the chunks are
    independent of each other and are filled on a thread pool (numpy releases
    the GIL in bulk draws and ufuncs). The bytes do not depend on the number
    of threads."""
    out = np.empty((rows, heads, d), dtype=np.uint16)

    def fill(c):
        r0, r1 = c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)
        z = _chunk_rng(key, c).standard_normal((r1 - r0, heads, d))
        if add is not None:
            z += add(r0, r1)
        out[r0:r1] = to_bf16_bits(z)

    n = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    if n <= 1:
        for c in range(n):
            fill(c)
    else:
        with cf.ThreadPoolExecutor(max_workers=min(n, _threads())) as ex:
            list(ex.map(fill, range(n)))
    return out


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _lowrank_structure(cfg, layer, frames, hq, hkv, d, rank=8):
    """Per-frame smooth field and its bases (the 'rank 8, amplitude 2' component)."""
    rng = rng_for(cfg, layer, STREAM_STRUCT)
    nf, hh, ww = frames
    a = rng.integers(0, 3, size=(nf, rank))
    b = rng.integers(0, 3, size=(nf, rank))
    phi = rng.uniform(0.0, 2.0 * math.pi, size=(nf, rank))

    def orthonormal_rows(n):
        g = rng.standard_normal((d, n))
        qm, _ = np.linalg.qr(g)
        return qm.T.copy()  # [n, d], orthonormal rows

    u = np.stack([orthonormal_rows(rank) for _ in range(hkv)])      # K bases
    w = np.stack([orthonormal_rows(rank) for _ in range(hkv)])      # V bases
    rot = []
    for _ in range(hq):
        qm, _ = np.linalg.qr(rng.standard_normal((rank, rank)))
        rot.append(qm)
    rot = np.stack(rot)                                             # [hq, r, r]
    return dict(a=a, b=b, phi=phi, u=u, w=w, rot=rot, frames=frames)


def _field(struct, t0, t1):
    """Unit-norm field c(t) for generation tokens [t0, t1): [n, rank] fp64."""
    nf, hh, ww = struct["frames"]
    t = np.arange(t0, t1)
    f = t // (hh * ww)
    y = (t // ww) % hh
    x = t % ww
    ang = 2.0 * math.pi * (struct["a"][f] * (y / hh)[:, None] + struct["b"][f] * (x / ww)[:, None]) \
        + struct["phi"][f]
    c = np.cos(ang)
    return c / np.linalg.norm(c, axis=1, keepdims=True)


def _fill_padding(case: Case, value):
    lay = case.layout
    if value is None:
        return
    bits = to_bf16_bits(np.float64(value)) if not isinstance(value, np.uint16) else value
    case.q[:, lay["q_valid"]:] = bits
    case.k[:, lay["kv_prefix_valid"]:lay["kv_prefix_len"]] = bits
    case.v[:, lay["kv_prefix_valid"]:lay["kv_prefix_len"]] = bits
    s0 = lay["kv_prefix_len"] + lay["kv_suffix_valid"]
    case.k[:, s0:] = bits
    case.v[:, s0:] = bits


def make_case(name="custom", *, cfg=0, layer=0, batch=1, hq=2, hkv=1, d=64, bq=64, bk=64,
              prefix=64, gen=448, sparsity=50, dist="normal", frames=None, scale=None,
              pad_fill=None, int_range=2) -> Case:
    """Build one case.

    ``dist``:
      * ``normal``  - Q, K, V i.i.d. N(0,1);
      * ``lowrank`` - N(0,1) plus the per-frame rank-8 field of amplitude 2
        (L2 norm 2 per token) on generation tokens; prefix tokens N(0,1);
      * ``int``     - integers uniform in [-int_range, int_range] (every pooled
        sum is exact in any precision);
      * ``cancel``  - every row of a block equal, with large components that
        cancel in the block-score dot product, so that an fp64 dot product is
        inexact near fp32 rounding boundaries.
    ``pad_fill``: value written into padding rows/keys (None keeps 0).
    """
    lay = make_layout(batch, hq, hkv, d, bq, bk, prefix, gen, scale)
    q = np.zeros((batch, lay["q_len"], hq, d), dtype=np.uint16)
    k = np.zeros((batch, lay["kv_len"], hkv, d), dtype=np.uint16)
    v = np.zeros((batch, lay["kv_len"], hkv, d), dtype=np.uint16)
    pl = lay["kv_prefix_len"]
    meta = dict(cfg=cfg, layer=layer, dist=dist)

    if dist in ("normal", "lowrank"):
        add = None
        if dist == "lowrank":
            if frames is None or frames[0] * frames[1] * frames[2] != gen:
                raise ValueError("lowrank needs frames with product == gen")
            st = _lowrank_structure(cfg, layer, frames, hq, hkv, d)
            grp = hq // hkv
            ub = st["u"][np.arange(hq) // grp]                              # U_{h//G}

            def add(which, t0, t1):
                c = _field(st, t0, t1)                                      # [n, 8]
                if which == "q":
                    rc = np.einsum("hrs,ns->nhr", st["rot"], c)             # R_h c
                    return 2.0 * np.einsum("nhr,hrd->nhd", rc, ub)
                basis = st["u"] if which == "k" else st["w"]
                return 2.0 * np.einsum("nr,grd->ngd", c, basis)
        for bi in range(batch):
            # key = (cfg, layer, stream, batch row, segment): segment 0 = generation
            # tokens, 1 = prefix tokens
            gk = lambda stream, seg: (cfg, layer, stream, bi, seg)
            q[bi, :gen] = _gen_rows(gk(STREAM_Q, 0), gen, hq, d, add and (lambda a, b: add("q", a, b)))
            k[bi, :prefix] = _gen_rows(gk(STREAM_K, 1), prefix, hkv, d)
            k[bi, pl:pl + gen] = _gen_rows(gk(STREAM_K, 0), gen, hkv, d,
                                           add and (lambda a, b: add("k", a, b)))
            v[bi, :prefix] = _gen_rows(gk(STREAM_V, 1), prefix, hkv, d)
            v[bi, pl:pl + gen] = _gen_rows(gk(STREAM_V, 0), gen, hkv, d,
                                           add and (lambda a, b: add("v", a, b)))
    elif dist == "int":
        r = rng_for(cfg, layer, STREAM_Q)
        q[:, :gen] = to_bf16_bits(r.integers(-int_range, int_range + 1, size=(batch, gen, hq, d)))
        for arr in (k, v):
            arr[:, :prefix] = to_bf16_bits(r.integers(-int_range, int_range + 1, size=(batch, prefix, hkv, d)))
            arr[:, pl:pl + gen] = to_bf16_bits(r.integers(-int_range, int_range + 1, size=(batch, gen, hkv, d)))
    elif dist == "cancel":
        r = rng_for(cfg, layer, STREAM_Q)
        if d % 2:
            raise ValueError("cancel needs an even head_dim")
        # Every row of a block is the same vector, so a block mean equals it.
        # Query vectors repeat each value in the pair (2m, 2m+1); about half of
        # the key blocks are antisymmetric in those pairs with huge values, so
        # their huge products cancel exactly while an fp64 running sum loses
        # the small ones. The other key blocks hold ordinary values.
        def mixed(shape):
            big = r.integers(-255, 256, size=shape) * np.exp2(r.integers(0, 40, size=shape).astype(np.float64))
            small = r.standard_normal(shape) * np.exp2(r.integers(-30, 1, size=shape).astype(np.float64))
            return np.where(r.random(shape) < 0.25, big, small)

        nq_blk, nk_blk = lay["q_len"] // bq, lay["kv_len"] // bk
        for bi in range(batch):
            half = mixed((nq_blk, hq, d // 2))
            qv = np.repeat(half, 2, axis=2)
            q[bi] = np.repeat(to_bf16_bits(qv), bq, axis=0)
            kv = mixed((nk_blk, hkv, d))
            anti = r.random((nk_blk, hkv)) < 0.5
            bigk = r.integers(-255, 256, size=(nk_blk, hkv, d // 2)) * np.exp2(
                r.integers(20, 40, size=(nk_blk, hkv, d // 2)).astype(np.float64))
            pair = np.stack([bigk, -bigk], axis=3).reshape(nk_blk, hkv, d)
            kv = np.where(anti[..., None], pair + np.where(np.arange(d) % 8 == 0, kv, 0.0), kv)
            k[bi] = np.repeat(to_bf16_bits(kv), bk, axis=0)
            v[bi] = to_bf16_bits(r.standard_normal((lay["kv_len"], hkv, d)))
        case = Case(name, lay, q, k, v, sparsity, meta)
        _zero_padding(case)
        _fill_padding(case, pad_fill)
        return case
    else:
        raise ValueError(f"unknown dist {dist!r}")

    case = Case(name, lay, q, k, v, sparsity, meta)
    _fill_padding(case, pad_fill)
    return case


def _zero_padding(case: Case):
    _fill_padding(case, 0.0)


def make_config(name: str, layer: int = 0, pad_fill=None) -> Case:
    """The named workload (for ``twostream``: layer ``layer`` of the schedule)."""
    c = dict(CONFIGS[name])
    cfg = c.pop("cfg")
    sparsity = c.pop("sparsity")
    layers = c.pop("layers", None)
    dense_layers = c.pop("dense_layers", None)
    if layers is not None:
        if not 0 <= layer < layers:
            raise ValueError("layer out of range")
        sparsity = 0 if layer < dense_layers else sparsity
    return make_case(name, cfg=cfg, layer=layer, sparsity=sparsity, pad_fill=pad_fill, **c)


def make_und_case(layer: int = 0, pad_fill=None, block: int = 128) -> Case:
    """The understanding stream of layer ``layer`` of the two-stream schedule,
    attending to itself causally: its 1,000 tokens padded to a block multiple
    are both the query rows and the keys (no prefix segment). The keys and
    values are the bytes of the two-stream case's prefix segment (same
    seeds); the queries are drawn as segment 2."""
    c = CONFIGS["twostream"]
    cfg, und, hq, hkv, d = c["cfg"], c["prefix"], c["hq"], c["hkv"], c["d"]
    lay = make_layout(1, hq, hkv, d, block, block, prefix=0, gen=und)
    q = np.zeros((1, lay["q_len"], hq, d), dtype=np.uint16)
    k = np.zeros((1, lay["kv_len"], hkv, d), dtype=np.uint16)
    v = np.zeros((1, lay["kv_len"], hkv, d), dtype=np.uint16)
    # key = (cfg, layer, stream, batch row, segment): segment 1 = the
    # understanding tokens as keys/values, 2 = the understanding queries
    q[0, :und] = _gen_rows((cfg, layer, STREAM_Q, 0, 2), und, hq, d)
    k[0, :und] = _gen_rows((cfg, layer, STREAM_K, 0, 1), und, hkv, d)
    v[0, :und] = _gen_rows((cfg, layer, STREAM_V, 0, 1), und, hkv, d)
    case = Case("und_causal", lay, q, k, v, 0, dict(cfg=cfg, layer=layer, dist="normal"))
    _fill_padding(case, pad_fill)
    return case


def sample_rows(case: Case, per_head: int, seed_layer: int = 0):
    """Query rows to check at full size: rows 0 and q_valid-1 plus uniform draws.

    Returns an int array [B, Hq, per_head] of row indices (< q_valid).
    """
    lay = case.layout
    rng = rng_for(case.meta.get("cfg", 0), seed_layer, STREAM_ROWS)
    qv = lay["q_valid"]
    out = np.empty((lay["batch"], lay["num_q_heads"], per_head), dtype=np.int64)
    for b in range(lay["batch"]):
        for h in range(lay["num_q_heads"]):
            extra = rng.integers(0, qv, size=max(0, per_head - 2))
            rows = np.concatenate([[0, qv - 1], extra])[:per_head]
            out[b, h] = rows
    return out
