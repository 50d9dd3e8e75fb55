"""ctypes binding of libspecverify (see include/specverify.h for the contract).

Argument marshalling only: shapes are checked, torch tensors are turned into
device pointers, and the call goes to the C ABI on the current HIP stream.
Every step of the verify path runs in the library's HIP kernels; there is no
fallback.  If the library has not been built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SV_F32 = 0
SV_BF16 = 1

_DEV_ERRORS = {0: "ok", 1: "token id out of range", 2: "uniform outside [0, 1)",
               3: "KV length negative or above the host bound", 4: "n_accepted outside [0, K]"}

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libspecverify error {code}: {message}")
        self.code = code


def lib():
    """Load libspecverify.so (raises if it is missing: there is no CPU path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m speculative_decoding_verify_04_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        h.sv_last_error.restype = ctypes.c_char_p
        h.sv_version.restype = i32
        h.spec_verify_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32,
                                                      ctypes.POINTER(sz)]
        h.spec_verify_attn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                       i32, i32, i32, i32, ctypes.c_float, vp, vp, sz, vp]
        h.spec_verify_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                               i32, i32, i32, i32, i32, i32, ctypes.c_float, vp,
                                               vp]
        h.spec_accept_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        h.spec_accept.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, ctypes.c_float,
                                  ctypes.c_float, i32, vp, vp, vp, vp, sz, vp]
        h.spec_compact_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                      i32, vp, vp]
        h.spec_verify_attn_ragged_workspace_size.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32,
                                                             ctypes.POINTER(sz)]
        h.spec_verify_attn_ragged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                              vp, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp,
                                              sz, vp]
        h.spec_accept_ragged_workspace_size.argtypes = [i32, vp, i32, ctypes.POINTER(sz)]
        h.spec_accept_ragged.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, i32,
                                         ctypes.c_float, ctypes.c_float, i32, vp, vp, vp, vp, sz,
                                         vp]
        h.spec_compact_kv_ragged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                             i32, i32, vp, vp]
        h.spec_accept_ex.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32,
                                     ctypes.c_float, ctypes.c_float, i32, i32, vp, vp, vp, vp, sz,
                                     vp]
        h.spec_accept_compact.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32,
                                          ctypes.c_float, ctypes.c_float, i32, i32, vp, vp, vp, vp,
                                          vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        h.spec_lm_head_parts.argtypes = [i32]
        h.spec_lm_head_stats.argtypes = [vp, vp, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp]
        h.spec_accept_prestats.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32,
                                           ctypes.c_float, ctypes.c_float, i32, i32, vp, vp, vp,
                                           vp, i32, vp, vp, vp, vp, sz, vp]
        h.sv_set_kernel_events.argtypes = [vp, vp]
        for f in ("sv_set_kernel_events", "spec_verify_attn_workspace_size", "spec_verify_attn",
                  "spec_verify_attn_noalloc",
                  "spec_accept_workspace_size", "spec_accept", "spec_compact_kv",
                  "spec_verify_attn_ragged_workspace_size", "spec_verify_attn_ragged",
                  "spec_accept_ragged_workspace_size", "spec_accept_ragged",
                  "spec_compact_kv_ragged", "spec_accept_ex", "spec_accept_compact",
                  "spec_lm_head_parts", "spec_lm_head_stats", "spec_accept_prestats"):
            getattr(h, f).restype = i32
        _lib = h
    return _lib


def sv_last_error() -> str:
    return lib().sv_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise SpecVerifyError(rc, sv_last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _host_i32(x) -> ctypes.Array:
    vals = [int(v) for v in (x.tolist() if hasattr(x, "tolist") else x)]
    return (ctypes.c_int32 * len(vals))(*vals)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def spec_verify_attn_workspace_size(B, K, Hq, Hkv, D, dtype, kv_len_host, prefix_len=0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().spec_verify_attn_workspace_size(B, K, Hq, Hkv, D, dtype,
                                                 _host_i32(kv_len_host), prefix_len,
                                                 ctypes.byref(n)))
    return n.value


def spec_verify_attn(q, k_cache, v_cache, kv_start, kv_len, kv_len_host, k_new, v_new, out, K,
                     k_prefix=None, v_prefix=None, softmax_scale=0.0, status=None,
                     workspace=None, check_rows=False):
    """Attention of the K+1 verify queries; writes ``out`` [B*(K+1), Hq, D].

    ``check_rows`` copies kv_start to the host to check every sequence's rows lie
    inside the cache (a synchronising check, off by default)."""
    R, Hq, D = q.shape
    _need(R % (K + 1) == 0, "q rows must be B*(K+1)")
    B = R // (K + 1)
    Hkv = k_cache.shape[1]
    dt = _kv_dtype(q)
    for t in (k_cache, v_cache, k_new, v_new, out):
        _need(t.dtype == q.dtype and t.is_cuda, "KV tensors must share q's dtype and device")
    _need(k_cache.shape[1:] == (Hkv, D) and v_cache.shape == k_cache.shape, "cache shape")
    _need(k_new.shape == (R, Hkv, D) and v_new.shape == (R, Hkv, D), "new K/V shape")
    _need(out.shape == q.shape, "out shape")
    _need(kv_start.dtype == torch.int64 and kv_start.shape == (B,), "kv_start [B] int64")
    _need(kv_len.dtype == torch.int32 and kv_len.shape == (B,), "kv_len [B] int32")
    hl = [int(v) for v in (kv_len_host.tolist() if hasattr(kv_len_host, "tolist") else kv_len_host)]
    _need(len(hl) == B, "kv_len_host has B entries")
    P = 0
    if k_prefix is not None:
        P = k_prefix.shape[0]
        _need(k_prefix.shape == (P, Hkv, D) and v_prefix.shape == (P, Hkv, D), "prefix shape")
    rows = k_cache.shape[0]
    if check_rows:
        ks = kv_start.cpu().tolist()
        for b in range(B):
            _need(0 <= ks[b] and ks[b] + hl[b] <= rows, f"cache rows of sequence {b} out of range")
    need = spec_verify_attn_workspace_size(B, K, Hq, Hkv, D, dt, hl, P)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace.numel() >= need, f"workspace needs {need} bytes")
    _check(lib().spec_verify_attn(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_start), _ptr(kv_len), _host_i32(hl),
        _ptr(k_new), _ptr(v_new), _ptr(k_prefix), _ptr(v_prefix), P, _ptr(out), B, K, Hq, Hkv,
        D, dt, float(softmax_scale), _ptr(status), _ptr(workspace), workspace.numel(),
        _stream(q)))
    return out


def spec_verify_attn_noalloc(q, k_cache, v_cache, kv_start, kv_len, kv_len_host, k_new, v_new,
                             out, K, k_prefix=None, v_prefix=None, softmax_scale=0.0,
                             status=None):
    """spec_verify_attn without a workspace: the library's fixed per-GPU scratch
    holds the counters and partial results (no device allocation here or in
    the library).  Calls that overlap on one GPU race on that scratch."""
    R, Hq, D = q.shape
    _need(R % (K + 1) == 0, "q rows must be B*(K+1)")
    B = R // (K + 1)
    Hkv = k_cache.shape[1]
    dt = _kv_dtype(q)
    for t in (k_cache, v_cache, k_new, v_new, out):
        _need(t.dtype == q.dtype and t.is_cuda, "KV tensors must share q's dtype and device")
    _need(k_cache.shape[1:] == (Hkv, D) and v_cache.shape == k_cache.shape, "cache shape")
    _need(k_new.shape == (R, Hkv, D) and v_new.shape == (R, Hkv, D), "new K/V shape")
    _need(out.shape == q.shape, "out shape")
    _need(kv_start.dtype == torch.int64 and kv_start.shape == (B,), "kv_start [B] int64")
    _need(kv_len.dtype == torch.int32 and kv_len.shape == (B,), "kv_len [B] int32")
    hl = [int(v) for v in (kv_len_host.tolist() if hasattr(kv_len_host, "tolist") else kv_len_host)]
    _need(len(hl) == B, "kv_len_host has B entries")
    P = 0
    if k_prefix is not None:
        P = k_prefix.shape[0]
        _need(k_prefix.shape == (P, Hkv, D) and v_prefix.shape == (P, Hkv, D), "prefix shape")
    _check(lib().spec_verify_attn_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_start), _ptr(kv_len), _host_i32(hl),
        _ptr(k_new), _ptr(v_new), _ptr(k_prefix), _ptr(v_prefix), P, _ptr(out), B, K, Hq, Hkv,
        D, dt, float(softmax_scale), _ptr(status), _stream(q)))
    return out


def spec_accept_workspace_size(B, K, V) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().spec_accept_workspace_size(B, K, V, ctypes.byref(n)))
    return n.value


def spec_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature,
                top_p, greedy, n_accepted, out_tokens, status=None, workspace=None, top_k=0):
    """One verify round of modified rejection sampling per sequence.

    Writes ``n_accepted`` [B] and ``out_tokens`` [B, K+1] (int32).  ``top_k`` > 0
    keeps the k largest logits of every row (and ties) before the nucleus."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    dt = _kv_dtype(target_logits)
    if draft_logits is not None:
        _need(draft_logits.shape == (B, K, V) and draft_logits.dtype == target_logits.dtype,
              "draft logits [B, K, V], same dtype as target")
    _need(draft_tokens.shape == (B, K) and draft_tokens.dtype == torch.int32, "draft tokens")
    if not greedy:
        _need(draft_logits is not None, "draft logits are required unless greedy")
        _need(u_accept.shape == (B, K) and u_accept.dtype == torch.float32, "u_accept [B, K]")
        _need(u_sample.shape == (B,) and u_sample.dtype == torch.float32, "u_sample [B]")
    _need(n_accepted.shape == (B,) and n_accepted.dtype == torch.int32, "n_accepted [B] int32")
    _need(out_tokens.shape == (B, K1) and out_tokens.dtype == torch.int32, "out_tokens")
    need = spec_accept_workspace_size(B, K, V)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=target_logits.device)
    _need(workspace.numel() >= need, f"workspace needs {need} bytes")
    if top_k:
        _check(lib().spec_accept_ex(
            _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens),
            _ptr(u_accept) if not greedy else None, _ptr(u_sample) if not greedy else None,
            None, None, B, K, V, float(temperature), float(top_p), int(top_k),
            int(bool(greedy)), _ptr(n_accepted), _ptr(out_tokens), _ptr(status),
            _ptr(workspace), workspace.numel(), _stream(target_logits)))
        return n_accepted, out_tokens
    _check(lib().spec_accept(
        _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens),
        _ptr(u_accept) if not greedy else None, _ptr(u_sample) if not greedy else None,
        B, K, V, float(temperature), float(top_p), int(bool(greedy)), _ptr(n_accepted),
        _ptr(out_tokens), _ptr(status), _ptr(workspace), workspace.numel(),
        _stream(target_logits)))
    return n_accepted, out_tokens


def spec_compact_kv(n_accepted, out_tokens, kv_len, kv_start, k_cache, v_cache, k_new, v_new,
                    tokens_packed, cu_tokens, status=None):
    """Padding-free compaction; updates kv_len, the caches, tokens_packed, cu_tokens."""
    B = n_accepted.shape[0]
    K = out_tokens.shape[1] - 1
    _, Hkv, D = k_cache.shape
    _need(out_tokens.shape == (B, K + 1), "out_tokens [B, K+1]")
    _need(kv_len.shape == (B,) and kv_len.dtype == torch.int32, "kv_len [B] int32")
    _need(kv_start.shape == (B,) and kv_start.dtype == torch.int64, "kv_start [B] int64")
    _need(k_new.shape == (B * (K + 1), Hkv, D) and v_new.shape == k_new.shape, "new K/V")
    _need(tokens_packed.numel() >= B * (K + 1) and cu_tokens.numel() == B + 1, "outputs")
    _check(lib().spec_compact_kv(
        _ptr(n_accepted), _ptr(out_tokens), _ptr(kv_len), _ptr(kv_start), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(tokens_packed), _ptr(cu_tokens), B, K,
        Hkv, D, _kv_dtype(k_cache), _ptr(status), _stream(k_cache)))
    return tokens_packed, cu_tokens


# ---------------------------------------------------------------- ragged draft lengths

def _cu_host(cu_q_host, B):
    hl = [int(v) for v in (cu_q_host.tolist() if hasattr(cu_q_host, "tolist") else cu_q_host)]
    _need(len(hl) == B + 1, "cu_q_host has B+1 entries")
    return hl


def spec_verify_attn_ragged_workspace_size(B, Hq, Hkv, D, dtype, kv_len_host, cu_q_host,
                                           prefix_len=0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().spec_verify_attn_ragged_workspace_size(
        B, Hq, Hkv, D, dtype, _host_i32(kv_len_host), _host_i32(_cu_host(cu_q_host, B)),
        prefix_len, ctypes.byref(n)))
    return n.value


def spec_verify_attn_ragged(q, k_cache, v_cache, kv_start, kv_len, kv_len_host, k_new, v_new,
                            out, cu_q, cu_q_host, k_prefix=None, v_prefix=None,
                            softmax_scale=0.0, status=None, workspace=None):
    """Attention of the K_b+1 verify queries of every sequence b, packed by the
    row offsets ``cu_q`` [B+1] (device int32; ``cu_q_host`` the same on the host);
    writes ``out`` [cu_q[B], Hq, D]."""
    B = kv_len.shape[0]
    hc = _cu_host(cu_q_host, B)
    R, Hq, D = q.shape
    _need(R == hc[B], "q rows must be cu_q[B]")
    Hkv = k_cache.shape[1]
    dt = _kv_dtype(q)
    for t in (k_cache, v_cache, k_new, v_new, out):
        _need(t.dtype == q.dtype and t.is_cuda, "KV tensors must share q's dtype and device")
    _need(k_cache.shape[1:] == (Hkv, D) and v_cache.shape == k_cache.shape, "cache shape")
    _need(k_new.shape == (R, Hkv, D) and v_new.shape == (R, Hkv, D), "new K/V shape")
    _need(out.shape == q.shape, "out shape")
    _need(cu_q.dtype == torch.int32 and cu_q.shape == (B + 1,), "cu_q [B+1] int32")
    _need(kv_start.dtype == torch.int64 and kv_start.shape == (B,), "kv_start [B] int64")
    _need(kv_len.dtype == torch.int32 and kv_len.shape == (B,), "kv_len [B] int32")
    hl = [int(v) for v in (kv_len_host.tolist() if hasattr(kv_len_host, "tolist") else kv_len_host)]
    _need(len(hl) == B, "kv_len_host has B entries")
    P = 0
    if k_prefix is not None:
        P = k_prefix.shape[0]
        _need(k_prefix.shape == (P, Hkv, D) and v_prefix.shape == (P, Hkv, D), "prefix shape")
    need = spec_verify_attn_ragged_workspace_size(B, Hq, Hkv, D, dt, hl, hc, P)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace.numel() >= need, f"workspace needs {need} bytes")
    _check(lib().spec_verify_attn_ragged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_start), _ptr(kv_len), _host_i32(hl),
        _ptr(k_new), _ptr(v_new), _ptr(k_prefix), _ptr(v_prefix), P, _ptr(out), _ptr(cu_q),
        _host_i32(hc), B, Hq, Hkv, D, dt, float(softmax_scale), _ptr(status), _ptr(workspace),
        workspace.numel(), _stream(q)))
    return out


def spec_accept_ragged_workspace_size(B, cu_q_host, V) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().spec_accept_ragged_workspace_size(B, _host_i32(_cu_host(cu_q_host, B)), V,
                                                   ctypes.byref(n)))
    return n.value


def spec_accept_ragged(target_logits, draft_logits, draft_tokens, u_accept, u_sample, cu_q,
                       cu_q_host, temperature, top_p, greedy, n_accepted, out_tokens,
                       status=None, workspace=None, top_k=0):
    """Modified rejection sampling with K_b drafts in sequence b: target rows
    cu_q[b]..cu_q[b+1]-1 of ``target_logits`` [cu_q[B], V]; draft rows, draft
    tokens and accept uniforms of b start at cu_q[b] - b.  Writes ``n_accepted``
    [B] and ``out_tokens`` [cu_q[B]] (b's K_b+1 entries from cu_q[b])."""
    B = n_accepted.shape[0]
    hc = _cu_host(cu_q_host, B)
    NT, V = target_logits.shape
    _need(NT == hc[B], "target rows must be cu_q[B]")
    ND = NT - B
    dt = _kv_dtype(target_logits)
    if draft_logits is not None:
        _need(draft_logits.shape == (ND, V) and draft_logits.dtype == target_logits.dtype,
              "draft logits [cu_q[B]-B, V], same dtype as target")
    _need(draft_tokens.shape == (ND,) and draft_tokens.dtype == torch.int32, "draft tokens")
    if not greedy:
        _need(draft_logits is not None, "draft logits are required unless greedy")
        _need(u_accept.shape == (ND,) and u_accept.dtype == torch.float32, "u_accept")
        _need(u_sample.shape == (B,) and u_sample.dtype == torch.float32, "u_sample [B]")
    _need(cu_q.dtype == torch.int32 and cu_q.shape == (B + 1,), "cu_q [B+1] int32")
    _need(n_accepted.dtype == torch.int32, "n_accepted [B] int32")
    _need(out_tokens.shape == (NT,) and out_tokens.dtype == torch.int32, "out_tokens [cu_q[B]]")
    need = spec_accept_ragged_workspace_size(B, hc, V)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=target_logits.device)
    _need(workspace.numel() >= need, f"workspace needs {need} bytes")
    if top_k:
        _check(lib().spec_accept_ex(
            _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens),
            _ptr(u_accept) if not greedy else None, _ptr(u_sample) if not greedy else None,
            _ptr(cu_q), _host_i32(hc), B, 0, V, float(temperature), float(top_p), int(top_k),
            int(bool(greedy)), _ptr(n_accepted), _ptr(out_tokens), _ptr(status),
            _ptr(workspace), workspace.numel(), _stream(target_logits)))
        return n_accepted, out_tokens
    _check(lib().spec_accept_ragged(
        _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens),
        _ptr(u_accept) if not greedy else None, _ptr(u_sample) if not greedy else None,
        _ptr(cu_q), _host_i32(hc), B, V, float(temperature), float(top_p), int(bool(greedy)),
        _ptr(n_accepted), _ptr(out_tokens), _ptr(status), _ptr(workspace), workspace.numel(),
        _stream(target_logits)))
    return n_accepted, out_tokens


def spec_compact_kv_ragged(n_accepted, out_tokens, kv_len, kv_start, k_cache, v_cache, k_new,
                           v_new, tokens_packed, cu_tokens, cu_q, status=None):
    """Padding-free compaction with K_b drafts in sequence b (rows packed by cu_q)."""
    B = n_accepted.shape[0]
    _, Hkv, D = k_cache.shape
    R = out_tokens.shape[0]
    _need(cu_q.dtype == torch.int32 and cu_q.shape == (B + 1,), "cu_q [B+1] int32")
    _need(kv_len.shape == (B,) and kv_len.dtype == torch.int32, "kv_len [B] int32")
    _need(kv_start.shape == (B,) and kv_start.dtype == torch.int64, "kv_start [B] int64")
    _need(k_new.shape == (R, Hkv, D) and v_new.shape == k_new.shape, "new K/V [cu_q[B], Hkv, D]")
    _need(tokens_packed.numel() >= R and cu_tokens.numel() == B + 1, "outputs")
    _check(lib().spec_compact_kv_ragged(
        _ptr(n_accepted), _ptr(out_tokens), _ptr(kv_len), _ptr(kv_start), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(tokens_packed), _ptr(cu_tokens), _ptr(cu_q),
        B, Hkv, D, _kv_dtype(k_cache), _ptr(status), _stream(k_cache)))
    return tokens_packed, cu_tokens


def spec_accept_compact(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature,
                        top_p, greedy, n_accepted, out_tokens, kv_len, kv_start, k_cache, v_cache,
                        k_new, v_new, tokens_packed, cu_tokens, status=None, workspace=None,
                        top_k=0, cu_q=None, cu_q_host=None):
    """spec_accept (or spec_accept_ragged with ``cu_q``/``cu_q_host``) and
    spec_compact_kv in one call: the sampler's kernels also append the accepted
    KV rows, advance ``kv_len`` and write ``tokens_packed`` and ``cu_tokens``.
    The tensors and their layouts are those of the two separate calls."""
    ragged = cu_q is not None
    B = n_accepted.shape[0]
    _, Hkv, D = k_cache.shape
    dt = _kv_dtype(target_logits)
    if ragged:
        hc = _cu_host(cu_q_host, B)
        NT, V = target_logits.shape
        _need(NT == hc[B], "target rows must be cu_q[B]")
        _need(cu_q.dtype == torch.int32 and cu_q.shape == (B + 1,), "cu_q [B+1] int32")
        _need(out_tokens.shape == (NT,) and out_tokens.dtype == torch.int32, "out_tokens [cu_q[B]]")
        K = 0
        R = NT
        need = spec_accept_ragged_workspace_size(B, hc, V)
        cu_dev, cu_host = _ptr(cu_q), _host_i32(hc)
    else:
        _, K1, V = target_logits.shape
        K = K1 - 1
        R = B * K1
        _need(out_tokens.shape == (B, K1) and out_tokens.dtype == torch.int32, "out_tokens")
        need = spec_accept_workspace_size(B, K, V)
        cu_dev, cu_host = None, None
    if not greedy:
        _need(draft_logits is not None, "draft logits are required unless greedy")
    _need(n_accepted.shape == (B,) and n_accepted.dtype == torch.int32, "n_accepted [B] int32")
    _need(kv_len.shape == (B,) and kv_len.dtype == torch.int32, "kv_len [B] int32")
    _need(kv_start.shape == (B,) and kv_start.dtype == torch.int64, "kv_start [B] int64")
    _need(k_new.shape == (R, Hkv, D) and v_new.shape == k_new.shape, "new K/V rows")
    _need(tokens_packed.numel() >= R and cu_tokens.numel() == B + 1, "outputs")
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=target_logits.device)
    _need(workspace.numel() >= need, f"workspace needs {need} bytes")
    _check(lib().spec_accept_compact(
        _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens),
        _ptr(u_accept) if not greedy else None, _ptr(u_sample) if not greedy else None,
        cu_dev, cu_host, B, K, V, float(temperature), float(top_p), int(top_k),
        int(bool(greedy)), _ptr(n_accepted), _ptr(out_tokens), _ptr(kv_len), _ptr(kv_start),
        _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), Hkv, D, _kv_dtype(k_cache),
        _ptr(tokens_packed), _ptr(cu_tokens), _ptr(status), _ptr(workspace), workspace.numel(),
        _stream(target_logits)))
    return n_accepted, out_tokens


def spec_lm_head_parts(V) -> int:
    n = lib().spec_lm_head_parts(int(V))
    if n < 0:
        _check(n)
    return n


def spec_lm_head_stats(hidden, weight, temperature, logits, part_max, part_sum):
    """LM head (logits = hidden @ weight^T, bf16 in, fp32 out) with every
    row's max and fp64 sum of exp((z - max)/T) over each part of 64 ids."""
    rows, H = hidden.shape
    V, H2 = weight.shape
    _need(H2 == H, "hidden [rows, H] and weight [V, H]")
    _need(hidden.dtype == torch.bfloat16 and weight.dtype == torch.bfloat16, "bf16 inputs")
    P = spec_lm_head_parts(V)
    _need(logits.shape == (rows, V) and logits.dtype == torch.float32, "logits [rows, V] fp32")
    _need(part_max.shape == (rows, P) and part_max.dtype == torch.float32, "part_max [rows, parts]")
    _need(part_sum.shape == (rows, P) and part_sum.dtype == torch.float64, "part_sum [rows, parts]")
    _check(lib().spec_lm_head_stats(_ptr(hidden), _ptr(weight), rows, H, V, float(temperature),
                                    _ptr(logits), _ptr(part_max), _ptr(part_sum),
                                    _stream(hidden)))
    return logits, part_max, part_sum


def spec_accept_prestats(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                         temperature, top_p, greedy, n_accepted, out_tokens, target_part_max,
                         target_part_sum, draft_part_max, draft_part_sum, status=None,
                         workspace=None, top_k=0):
    """spec_accept with the rows' statistics from spec_lm_head_stats (used by
    stochastic calls without a filter; the segment pass is skipped)."""
    B, K1, V = target_logits.shape
    K = K1 - 1
    dt = _kv_dtype(target_logits)
    P = target_part_max.shape[-1]
    _need(target_part_max.shape == (B * K1, P) and target_part_sum.shape == (B * K1, P),
          "target statistics [B*(K+1), parts]")
    if draft_part_max is not None:
        _need(draft_part_max.shape == (B * K, P) and draft_part_sum.shape == (B * K, P),
              "draft statistics [B*K, parts]")
    _need(n_accepted.shape == (B,) and out_tokens.shape == (B, K1), "outputs")
    need = spec_accept_workspace_size(B, K, V)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=target_logits.device)
    _need(workspace.numel() >= need, f"workspace needs {need} bytes")
    _check(lib().spec_accept_prestats(
        _ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens),
        _ptr(u_accept) if not greedy else None, _ptr(u_sample) if not greedy else None,
        None, None, B, K, V, float(temperature), float(top_p), int(top_k), int(bool(greedy)),
        _ptr(target_part_max), _ptr(target_part_sum), _ptr(draft_part_max), _ptr(draft_part_sum),
        P, _ptr(n_accepted), _ptr(out_tokens), _ptr(status), _ptr(workspace), workspace.numel(),
        _stream(target_logits)))
    return n_accepted, out_tokens


def sv_set_kernel_events(start: Optional[int], stop: Optional[int]) -> None:
    """Record hipEvent handles ``start``/``stop`` around the split-K chunk kernel of
    later spec_verify_attn calls on this thread (None turns it off)."""
    _check(lib().sv_set_kernel_events(ctypes.c_void_p(start) if start else None,
                                      ctypes.c_void_p(stop) if stop else None))


def device_error_name(code: int) -> str:
    return _DEV_ERRORS.get(int(code), f"unknown device error {code}")
