"""The allocation-free attention entry point (spec_verify_attn_noalloc) against
spec_verify_attn and the oracle, through the C ABI (needs an MI355X).

Two calls in a row share the library's fixed scratch, the second with a
smaller problem of another shape (fewer sequences, GQA, shorter caches), so
its counter layout and partial results overlap the first call's leftovers.
Each output must equal spec_verify_attn's bit for bit (same kernels, same
plan) and the oracle's within the bf16 bar.  Sizes beyond the scratch are
rejected before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import specref as R
from speculative_decoding_verify_04_amd import api
from speculative_decoding_verify_04_amd import workloads as W
from speculative_decoding_verify_04_amd.devio import to_device

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _errors(o, ref):
    num = np.abs(o - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return num / den


def _both(w):
    c = w.cfg
    t = to_device(w, DEV)
    t.status.zero_()
    api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, w.kv_len, t.k_new,
                         t.v_new, t.out, c.K, k_prefix=t.k_prefix, v_prefix=t.v_prefix,
                         status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0
    o_ws = t.out.float().cpu().numpy().astype(np.float64)
    out2 = torch.full_like(t.out, float("nan"))
    api.spec_verify_attn_noalloc(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, w.kv_len,
                                 t.k_new, t.v_new, out2, c.K, k_prefix=t.k_prefix,
                                 v_prefix=t.v_prefix, status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0
    return o_ws, out2.float().cpu().numpy().astype(np.float64)


def test_noalloc_matches_workspace_entry_point_twice():
    first = W.CONFIGS["bass_b8k5"]
    # (32 query columns per kv head: the grouped-head kernel over the even
    # split, whose arrival counters are in the fixed scratch too)
    second = W.small_variant(W.CONFIGS["gqa_b64k8"], B=3, K=7, Hq=8, Hkv=2, len_lo=50,
                             len_hi=700, V=64)
    for cfg, seed in ((first, 1), (second, 2)):
        print(f"[noalloc] B={cfg.B} K={cfg.K} Hq={cfg.Hq} Hkv={cfg.Hkv}", flush=True)
        w = W.make_workload(cfg, sub_seed=seed)
        o_ws, o_na = _both(w)
        assert np.array_equal(o_ws, o_na), "noalloc output differs from the workspace call"
        ref = R.workload_attn(w)
        assert _errors(o_na, ref).max() <= 1e-2


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = api.lib()
    small = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    p = ctypes.c_void_p(small.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    # 8192-row shared prefix over 64 sequences of 5 queries, 32 heads: the
    # prefix partials alone take 8 x 32 x 320 x 128 x 4 bytes = 40 MiB
    B, K, H, D, P = 64, 4, 32, 128, 8192
    L = (ctypes.c_int32 * B)(*([16] * B))
    rc = lib.spec_verify_attn_noalloc(p, p, p, p, p, L, p, p, p, p, P, p, B, K, H, H, D,
                                      api.SV_BF16, ctypes.c_float(0.0), None, stream)
    assert rc == -2, rc
    assert b"scratch" in lib.sv_last_error()
    # more arrival counters than the scratch holds: B * Hkv = 2048 * 64
    B, H = 2048, 64
    L = (ctypes.c_int32 * B)(*([16] * B))
    rc = lib.spec_verify_attn_noalloc(p, p, p, p, p, L, p, p, None, None, 0, p, B, 0, H, H, 64,
                                      api.SV_BF16, ctypes.c_float(0.0), None, stream)
    assert rc == -2, rc
    torch.cuda.synchronize()
