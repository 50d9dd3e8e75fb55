"""ctypes wrapper around the C oracle (test infrastructure only).

Every function takes plain numpy arrays (host memory) and returns numpy arrays.
bf16 tensors are passed as their uint16 bit patterns.  Nothing here imports or
calls the GPU library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

F32 = 0
BF16 = 1

_lib = None


def load(path: str):
    """Load an oracle build from ``path`` (the tests also load mutated builds)."""
    h = ctypes.CDLL(path)
    h.specref_verify_attn.restype = ctypes.c_int
    h.specref_accept.restype = ctypes.c_int
    h.specref_compact_kv.restype = ctypes.c_int
    h.specref_row_dist.restype = ctypes.c_int
    h.specref_lm_head.restype = ctypes.c_int
    h.specref_row_stats.restype = ctypes.c_int
    return h


def lib(override=None):
    global _lib
    if override is not None:
        return override
    if _lib is None:
        _lib = load(_build.build(force=False))
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _kv_dtype(a) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"KV arrays must be bf16 bits (uint16) or float32, got {a.dtype}")


def verify_attn(q, k_cache, v_cache, kv_start, kv_len, k_new, v_new, B, K, Hq, Hkv, D,
                k_prefix=None, v_prefix=None, scale=0.0, sel_rows=None, sel_heads=None,
                lib_=None):
    """fp64 attention of the K+1 verify queries.

    Returns [B*(K+1), Hq, D] float64, or [n_sel, D] for the listed (row, head) pairs.
    """
    dt = _kv_dtype(q)
    store = np.uint16 if dt == BF16 else np.float32
    arrs = [_c(x, store) for x in (q, k_cache, v_cache, k_new, v_new)]
    kp = None if k_prefix is None else _c(k_prefix, store)
    vp = None if v_prefix is None else _c(v_prefix, store)
    P = 0 if kp is None else int(kp.shape[0])
    ks, kl = _c(kv_start, np.int64), _c(kv_len, np.int32)
    if sel_rows is None:
        out = np.zeros((B * (K + 1), Hq, D), dtype=np.float64)
        sr = sh = None
        n_sel = -1
    else:
        sr, sh = _c(sel_rows, np.int32), _c(sel_heads, np.int32)
        n_sel = int(sr.shape[0])
        out = np.zeros((n_sel, D), dtype=np.float64)
    rc = lib(lib_).specref_verify_attn(
        _p(arrs[0]), _p(arrs[1]), _p(arrs[2]), _p(ks), _p(kl), _p(arrs[3]), _p(arrs[4]),
        _p(kp), _p(vp), ctypes.c_int(P), B, K, Hq, Hkv, D, dt, ctypes.c_double(scale),
        _p(sr), _p(sh), ctypes.c_int(n_sel), _p(out))
    if rc:
        raise ValueError(f"specref_verify_attn failed: {rc}")
    return out


def accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature,
           top_p, greedy=False, lib_=None, top_k=0):
    """One verify round of modified rejection sampling per sequence.

    Returns a dict with n_accepted [B], out_tokens [B, K+1], q_tok/p_tok [B, K],
    flag_pos [B], n_decisions, n_flagged.  ``temperature`` and ``top_p`` are
    rounded to float32 first, as the GPU library receives them; ``top_k`` > 0
    keeps the k most probable tokens (and ties) before the nucleus.
    """
    tl = _c(target_logits, np.float32)
    B, K1, V = tl.shape
    K = K1 - 1
    dl = None if draft_logits is None else _c(draft_logits, np.float32)
    if dl is None and not greedy:
        raise ValueError("draft logits are required unless greedy")
    dtok = _c(draft_tokens, np.int32).reshape(B, K)
    ua = _c(u_accept, np.float32).reshape(B, K)
    us = _c(u_sample, np.float32).reshape(B)
    n = np.zeros(B, np.int32)
    out = np.zeros((B, K + 1), np.int32)
    qt = np.zeros((B, K), np.float64)
    pt = np.zeros((B, K), np.float64)
    fp = np.zeros(B, np.int32)
    nd = ctypes.c_int64(0)
    nf = ctypes.c_int64(0)
    rc = lib(lib_).specref_accept(
        _p(tl), _p(dl), _p(dtok), _p(ua), _p(us), B, K, V,
        ctypes.c_double(float(np.float32(temperature))),
        ctypes.c_double(float(np.float32(top_p))), int(top_k), int(bool(greedy)),
        _p(n), _p(out), _p(qt), _p(pt), _p(fp), ctypes.byref(nd), ctypes.byref(nf))
    if rc:
        raise ValueError(f"specref_accept failed: {rc}")
    return {"n_accepted": n, "out_tokens": out, "q_tok": qt, "p_tok": pt, "flag_pos": fp,
            "n_decisions": int(nd.value), "n_flagged": int(nf.value)}


def row_dist(z, temperature, top_p, top_k=0, lib_=None):
    """The modified distribution pi' of one row of logits z [V] (temperature,
    top-k, nucleus), in float64; ``temperature`` and ``top_p`` are rounded to
    float32 first, as the GPU library receives them."""
    zz = _c(z, np.float32).reshape(-1)
    V = int(zz.shape[0])
    pi = np.zeros(V, np.float64)
    amb = ctypes.c_int32(0)
    rc = lib(lib_).specref_row_dist(
        _p(zz), V, ctypes.c_double(float(np.float32(temperature))), int(top_k),
        ctypes.c_double(float(np.float32(top_p))), _p(pi), ctypes.byref(amb))
    if rc:
        raise ValueError(f"specref_row_dist failed: {rc}")
    return pi


def lm_head(hidden, weight, lib_=None):
    """LM head: z[r][v] = sum_h hidden[r][h] * weight[v][h] in fp64, from bf16
    (uint16 bits) or float32 inputs of the same type.  Returns [rows, V] float64."""
    dt = _kv_dtype(hidden)
    store = np.uint16 if dt == BF16 else np.float32
    hd, wt = _c(hidden, store), _c(weight, store)
    rows, H = hd.shape
    V, H2 = wt.shape
    if H2 != H:
        raise ValueError("hidden [rows, H] and weight [V, H]")
    out = np.zeros((rows, V), np.float64)
    rc = lib(lib_).specref_lm_head(_p(hd), _p(wt), dt, rows, H, V, _p(out))
    if rc:
        raise ValueError(f"specref_lm_head failed: {rc}")
    return out


def row_stats(z, temperature, lib_=None):
    """Per row of fp32 logits z [rows, V]: (m, S) with m = max z and
    S = sum exp((z - m) / T), both float64 [rows]."""
    zz = _c(z, np.float32)
    rows, V = zz.shape
    m = np.zeros(rows, np.float64)
    S = np.zeros(rows, np.float64)
    for r in range(rows):
        mr, sr = ctypes.c_double(0.0), ctypes.c_double(0.0)
        rc = lib(lib_).specref_row_stats(_p(zz[r]), V, ctypes.c_double(float(temperature)),
                                         ctypes.byref(mr), ctypes.byref(sr))
        if rc:
            raise ValueError(f"specref_row_stats failed: {rc}")
        m[r], S[r] = mr.value, sr.value
    return m, S


def compact_kv(n_accepted, out_tokens, kv_len, kv_start, k_cache, v_cache, k_new, v_new,
               K, Hkv, D, lib_=None):
    """Padding-free compaction.  Returns (tokens_packed, cu_tokens, kv_len, k_cache,
    v_cache) as new arrays; the inputs are not modified."""
    n = _c(n_accepted, np.int32)
    B = int(n.shape[0])
    ot = _c(out_tokens, np.int32)
    kl = _c(kv_len, np.int32).copy()
    ks = _c(kv_start, np.int64)
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    kn = np.ascontiguousarray(k_new)
    vn = np.ascontiguousarray(v_new)
    es = kc.dtype.itemsize
    packed = np.full(B * (K + 1), -1, np.int32)
    cu = np.zeros(B + 1, np.int32)
    rc = lib(lib_).specref_compact_kv(_p(n), _p(ot), _p(kl), _p(ks), _p(kc), _p(vc), _p(kn),
                                  _p(vn), _p(packed), _p(cu), B, K, Hkv, D, es)
    if rc:
        raise ValueError(f"specref_compact_kv failed: {rc}")
    return packed, cu, kl, kc, vc


# ---------------------------------------------------------------- ragged draft lengths
#
# "EMS-SD: Efficient Multi-sample Speculative Decoding" (abstract): samples may
# carry different numbers of prediction tokens, without padding.  Sequences
# are independent in every operation, so sequence b of a ragged call is the
# uniform problem with one sequence and K = K_b on its own packed rows
# cu_q[b] .. cu_q[b+1]-1; these wrappers apply the uniform oracle that way.

def verify_attn_ragged(q, k_cache, v_cache, kv_start, kv_len, k_new, v_new, cu_q, Hq, Hkv, D,
                       k_prefix=None, v_prefix=None, scale=0.0, lib_=None):
    """fp64 attention with K_b + 1 queries in sequence b; returns [cu_q[B], Hq, D]."""
    cu = np.asarray(cu_q, dtype=np.int64)
    B = cu.shape[0] - 1
    out = np.zeros((int(cu[B]), Hq, D), dtype=np.float64)
    for b in range(B):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        out[r0:r1] = verify_attn(q[r0:r1], k_cache, v_cache, np.asarray(kv_start)[b:b + 1],
                                 np.asarray(kv_len)[b:b + 1], k_new[r0:r1], v_new[r0:r1], 1,
                                 r1 - r0 - 1, Hq, Hkv, D, k_prefix=k_prefix, v_prefix=v_prefix,
                                 scale=scale, lib_=lib_)
    return out


def accept_ragged(target_logits, draft_logits, draft_tokens, u_accept, u_sample, cu_q,
                  temperature, top_p, greedy=False, lib_=None, top_k=0):
    """Modified rejection sampling with K_b drafts in sequence b.  Target rows of b
    are cu_q[b] .. cu_q[b+1]-1; its draft rows, drafts and accept uniforms start
    at cu_q[b] - b.  Returns n_accepted [B], out_tokens [cu_q[B]] (b's K_b + 1
    entries from cu_q[b]), flag_pos [B], n_decisions, n_flagged."""
    cu = np.asarray(cu_q, dtype=np.int64)
    B = cu.shape[0] - 1
    V = target_logits.shape[-1]
    n = np.zeros(B, np.int32)
    out = np.zeros(int(cu[B]), np.int32)
    fp = np.zeros(B, np.int32)
    nd = nf = 0
    for b in range(B):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        k = r1 - r0 - 1
        d0 = r0 - b
        dl = None if (greedy and draft_logits is None) else \
            np.asarray(draft_logits)[d0:d0 + k].reshape(1, k, V)
        a = accept(np.asarray(target_logits)[r0:r1].reshape(1, k + 1, V), dl,
                   np.asarray(draft_tokens)[d0:d0 + k].reshape(1, k),
                   np.asarray(u_accept)[d0:d0 + k].reshape(1, k),
                   np.asarray(u_sample)[b:b + 1], temperature, top_p, greedy, lib_=lib_,
                   top_k=top_k)
        n[b] = a["n_accepted"][0]
        out[r0:r1] = a["out_tokens"][0]
        fp[b] = a["flag_pos"][0]
        nd += a["n_decisions"]
        nf += a["n_flagged"]
    return {"n_accepted": n, "out_tokens": out, "flag_pos": fp, "n_decisions": nd,
            "n_flagged": nf}


def compact_kv_ragged(n_accepted, out_tokens, kv_len, kv_start, k_cache, v_cache, k_new, v_new,
                      cu_q, Hkv, D, lib_=None):
    """Padding-free compaction with K_b drafts in sequence b: the uniform
    compaction of each sequence on its own rows, the packed tokens placed at
    the exclusive scan of the emitted counts.  Returns (tokens_packed,
    cu_tokens, kv_len, k_cache, v_cache) as new arrays."""
    cu = np.asarray(cu_q, dtype=np.int64)
    B = cu.shape[0] - 1
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    kl = np.array(kv_len, dtype=np.int32, copy=True)
    packed = np.full(int(cu[B]), -1, np.int32)
    cut = np.zeros(B + 1, np.int32)
    for b in range(B):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        k = r1 - r0 - 1
        pk, c1, l1, kc, vc = compact_kv(np.asarray(n_accepted)[b:b + 1],
                                        np.asarray(out_tokens)[r0:r1].reshape(1, k + 1),
                                        kl[b:b + 1], np.asarray(kv_start)[b:b + 1], kc, vc,
                                        k_new[r0:r1], v_new[r0:r1], k, Hkv, D, lib_=lib_)
        e = int(c1[1])
        packed[cut[b]:cut[b] + e] = pk[:e]
        cut[b + 1] = cut[b] + e
        kl[b] = l1[0]
    return packed, cut, kl, kc, vc


def workload_attn(w, sel_rows=None, sel_heads=None):
    """Oracle attention on a workload object from the shared input generator."""
    c = w.cfg
    return verify_attn(w.q, w.k_cache, w.v_cache, w.kv_start, w.kv_len, w.k_new, w.v_new,
                       c.B, c.K, c.Hq, c.Hkv, c.D, k_prefix=w.k_prefix,
                       v_prefix=w.v_prefix, sel_rows=sel_rows, sel_heads=sel_heads)


def workload_accept(w):
    c = w.cfg
    return accept(w.target_logits, None if c.greedy else w.draft_logits, w.draft_tokens,
                  w.u_accept, w.u_sample, c.temperature, c.top_p, c.greedy)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact conversion of bf16 bit patterns to float64."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def kv_to_f64(a: np.ndarray) -> np.ndarray:
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecref.so")
