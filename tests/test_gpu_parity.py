"""GPU path vs the CPU oracle, through the C ABI (needs an MI355X).

Bars:
  * attention: per output row, max_d |o - o_ref| <= tol * max_d |o_ref|, with
    tol = 1e-2 for bf16 inputs (fp32 accumulation) and 1e-5 for fp32.
  * sampler: n_accepted and out_tokens bit-exact, except that a decision the
    oracle flags as ambiguous (|u p - q| < 1e-6 p, a draw or nucleus boundary
    within 1e-12 of its edge) releases that sequence from that position on;
    flagged decisions must stay below 0.01% of all decisions.
  * compaction: bit-exact.
"""
import os

import numpy as np
import pytest
import torch

from oracle import specref as R
from speculative_decoding_verify_04_amd import api
from speculative_decoding_verify_04_amd import workloads as W
from speculative_decoding_verify_04_amd.devio import kv_tensor, ragged_to_device, to_device

import pins

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- helpers

def run_attn(w, t, scale=0.0):
    c = w.cfg
    t.status.zero_()
    api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, w.kv_len, t.k_new,
                         t.v_new, t.out, c.K, k_prefix=t.k_prefix, v_prefix=t.v_prefix,
                         softmax_scale=scale, status=t.status, check_rows=True)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0
    return t.out.float().cpu().numpy().astype(np.float64)


def attn_errors(o, ref):
    """Row-relative infinity-norm error per output row."""
    num = np.abs(o - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return num / den


def attn_tol(cfg):
    return 1e-5 if cfg.kv_dtype == W.F32 else 1e-2


def run_accept(w, t, greedy=None):
    c = w.cfg
    g = c.greedy if greedy is None else greedy
    t.status.zero_()
    api.spec_accept(t.target_logits, None if g else t.draft_logits, t.draft_tokens, t.u_accept,
                    t.u_sample, c.temperature, c.top_p, g, t.n_accepted, t.out_tokens,
                    status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0, api.device_error_name(int(t.status.item()))
    return t.n_accepted.cpu().numpy(), t.out_tokens.cpu().numpy()


def check_flagged_valid(n_b, toks_b, zt_b, zd_b, drafts_b, T, top_p, top_k=0):
    """A sequence released from the bit-exact comparison by a flagged decision
    must still be a valid round: its first n_b tokens are the drafts, the token
    at n_b has positive weight under the distribution it is drawn from --
    (q'_n - p'_n)_+ after a rejection (q'_n when that has no mass), q'_K for the
    bonus -- and the rest is -1.  ("Modified rejection sampling": an id of
    weight zero has probability zero.)"""
    K = drafts_b.shape[0]
    assert 0 <= n_b <= K
    assert np.array_equal(toks_b[:n_b], drafts_b[:n_b])
    assert np.all(toks_b[n_b + 1:] == -1)
    tok = int(toks_b[n_b])
    V = zt_b.shape[-1]
    assert 0 <= tok < V
    q = R.row_dist(zt_b[n_b], T, top_p, top_k)
    if n_b == K:
        assert q[tok] > 0.0, ("bonus token of zero weight", tok)
        return
    p = R.row_dist(zd_b[n_b], T, top_p, top_k)
    w = np.maximum(q - p, 0.0)
    if w.sum() > 0.0:
        assert w[tok] > 0.0, ("residual token of zero weight", n_b, tok)
    else:
        assert q[tok] > 0.0, ("fallback token of zero weight", n_b, tok)


def rows_of(w, top_k=0):
    """The inputs check_flagged_valid needs, from a workload."""
    c = w.cfg
    return (w.target_logits, None if c.greedy else w.draft_logits, w.draft_tokens,
            c.temperature, c.top_p, top_k)


def compare_accept(n, toks, ref, K, rows=None):
    """Bit-exact outside flagged decisions; a flagged sequence must agree before
    its flag and, given its inputs ``rows`` = (target logits, draft logits,
    drafts, T, top_p, top_k), be a valid round (check_flagged_valid).
    Returns (#sequences compared fully)."""
    full = 0
    for b in range(n.shape[0]):
        f, nr = int(ref["flag_pos"][b]), int(ref["n_accepted"][b])
        if f < 0 or f > nr:
            assert n[b] == nr, (b, n[b], nr)
            assert np.array_equal(toks[b], ref["out_tokens"][b]), (b, toks[b], ref["out_tokens"][b])
            full += 1
        else:
            assert n[b] >= f, (b, n[b], f)
            assert np.array_equal(toks[b, :f], ref["out_tokens"][b, :f])
            if rows is not None:
                zt, zd, dr, T, tp, tk = rows
                check_flagged_valid(int(n[b]), toks[b], zt[b], None if zd is None else zd[b],
                                    dr[b], T, tp, tk)
    return full


class FlagBudget:
    def __init__(self):
        self.decisions = 0
        self.flagged = 0

    def add(self, ref):
        self.decisions += ref["n_decisions"]
        self.flagged += ref["n_flagged"]

    def check(self):
        assert self.decisions > 0
        assert self.flagged <= 1e-4 * self.decisions, (self.flagged, self.decisions)


def gpu_sampler(zt, zd, tok, ua, us, T, top_p, greedy, top_k=0):
    B, K1, V = zt.shape
    K = K1 - 1
    dev = DEV
    n = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, K1), dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    api.spec_accept(torch.from_numpy(np.ascontiguousarray(zt)).to(dev),
                    None if greedy else torch.from_numpy(np.ascontiguousarray(zd)).to(dev),
                    torch.from_numpy(np.ascontiguousarray(tok, np.int32)).to(dev),
                    torch.from_numpy(np.ascontiguousarray(ua, np.float32)).to(dev),
                    torch.from_numpy(np.ascontiguousarray(us, np.float32)).to(dev),
                    T, top_p, greedy, n, out, status=st, top_k=top_k)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return {"n_accepted": n.cpu().numpy(), "out_tokens": out.cpu().numpy()}


# ---------------------------------------------------------------- attention: small shapes

SMALL_ATTN = {
    "tiny_fp32": W.CONFIGS["tiny_fp32"],
    "fp32_d64_prefix": W.small_variant(W.CONFIGS["prefix_b32k4"], kv_dtype=W.F32, B=3, Hq=4,
                                       Hkv=2, D=64, prefix_len=300, len_lo=0, len_hi=90, V=64),
    "bf16_mha_d128": W.small_variant(W.CONFIGS["bass_b8k5"], B=4, Hq=4, Hkv=4, len_lo=0,
                                     len_hi=700, V=64),
    "bf16_mha_d64": W.small_variant(W.CONFIGS["bass_b8k5"], B=3, Hq=3, Hkv=3, D=64, len_lo=1,
                                    len_hi=300, V=64),
    "bf16_gqa_k8": W.small_variant(W.CONFIGS["gqa_b64k8"], B=5, Hq=8, Hkv=2, len_lo=100,
                                   len_hi=900, V=64),
    "bf16_gqa_g8_k7": W.small_variant(W.CONFIGS["gqa_b64k8"], B=2, K=7, Hq=16, Hkv=2, D=64,
                                      len_lo=10, len_hi=200, V=64),
    "bf16_prefix": W.small_variant(W.CONFIGS["prefix_b32k4"], B=6, Hq=4, Hkv=4, prefix_len=700,
                                   len_lo=0, len_hi=40, V=64),
    "bf16_prefix_gqa_many_cols": W.small_variant(W.CONFIGS["prefix_b32k4"], B=60, K=4, Hq=8,
                                                 Hkv=2, prefix_len=1100, len_lo=0, len_hi=20,
                                                 V=64),
    # prefix kernel edge cases: head dim 64 (register-staged tiles), a prefix
    # shorter than one 64-key half, a second chunk ending inside the second
    # half of its only tile, and prefix chunks filled exactly
    "bf16_prefix_d64": W.small_variant(W.CONFIGS["prefix_b32k4"], B=5, Hq=4, Hkv=2, D=64,
                                       prefix_len=333, len_lo=0, len_hi=50, V=64),
    "bf16_prefix_tiny": W.small_variant(W.CONFIGS["prefix_b32k4"], B=3, Hq=2, Hkv=2,
                                        prefix_len=5, len_lo=0, len_hi=30, V=64),
    "bf16_prefix_half_tail": W.small_variant(W.CONFIGS["prefix_b32k4"], B=4, Hq=4, Hkv=4,
                                             prefix_len=1124, len_lo=0, len_hi=30, V=64),
    "bf16_prefix_exact_chunks": W.small_variant(W.CONFIGS["prefix_b32k4"], B=2, Hq=2, Hkv=2,
                                                prefix_len=2048, len_lo=0, len_hi=10, V=64),
    "bf16_k0_single_query": W.small_variant(W.CONFIGS["bass_b8k5"], K=0, B=3, Hq=2, Hkv=2,
                                            len_lo=0, len_hi=200, V=64),
    "bf16_all_empty_cache": W.small_variant(W.CONFIGS["bass_b8k5"], B=4, Hq=2, Hkv=2, len_lo=0,
                                            len_hi=0, V=64),
    "chinchilla_heads8": W.small_variant(W.CONFIGS["chinchilla_b1k4"], Hq=8, Hkv=8, V=64),
    # many (sequence, chunk, head) work items of unequal chunk counts
    "bf16_many_items": W.small_variant(W.CONFIGS["bass_b8k5"], B=16, Hq=8, Hkv=8, len_lo=1,
                                       len_hi=2500, V=64),
    "bf16_gqa_many_items": W.small_variant(W.CONFIGS["gqa_b64k8"], B=24, K=5, Hq=8, Hkv=2,
                                           len_lo=700, len_hi=3000, V=64),
    # grouped heads over the even split of the slices, with a shared prefix
    "bf16_prefix_gqa_even": W.small_variant(W.CONFIGS["prefix_b32k4"], B=6, K=4, Hq=8, Hkv=2,
                                            prefix_len=700, len_lo=100, len_hi=600, V=64),
    # 64 query columns per kv head: four column tiles, the fourth read from
    # the query item's second half; short and long sequences side by side
    "bf16_gqa_four_tiles": W.small_variant(W.CONFIGS["gqa_b64k8"], len_kind="uniform", B=11, K=7,
                                           Hq=16, Hkv=2, len_lo=0, len_hi=1500, V=64),
    # more work items than workgroups resident at once (one chunk each)
    "bf16_more_items_than_resident": W.small_variant(W.CONFIGS["bass_b8k5"], B=600, K=3, Hq=2,
                                                     Hkv=2, len_lo=0, len_hi=80, V=64),
    # one long sequence: each (sequence, head) is cut into hundreds of chunks
    "bf16_long_single": W.small_variant(W.CONFIGS["chinchilla_b1k4"], Hq=2, Hkv=2,
                                        fixed_lens=(120000,), len_lo=120000, len_hi=120000,
                                        V=64),
}


@pytest.mark.parametrize("name", list(SMALL_ATTN))
def test_attention_small(name):
    cfg = SMALL_ATTN[name]
    say(f"[attn small] {name}")
    w = W.make_workload(cfg, sub_seed=21)
    t = to_device(w, DEV)
    o = run_attn(w, t)
    ref = R.workload_attn(w)
    err = attn_errors(o, ref)
    assert np.isfinite(o).all()
    assert err.max() <= attn_tol(cfg), (name, float(err.max()))


# shapes that run the grouped-head kernel (D = 128, more than 16 query columns
# per kv head); by default over the even split of the slices
GQA_RING = ["bf16_gqa_k8", "bf16_gqa_many_items", "bf16_prefix_gqa_even",
            "bf16_prefix_gqa_many_cols", "bf16_gqa_four_tiles"]


@pytest.mark.parametrize("name", GQA_RING)
def test_attention_gqa_per_sequence_chunks(name, monkeypatch):
    """The grouped-head kernel over per-sequence chunks (SPECVERIFY_SK_CHUNKS=1)
    instead of the even split of the slices: the same oracle bar."""
    cfg = SMALL_ATTN[name]
    w = W.make_workload(cfg, sub_seed=21)
    t = to_device(w, DEV)
    monkeypatch.setenv("SPECVERIFY_SK_CHUNKS", "1")
    o = run_attn(w, t)
    ref = R.workload_attn(w)
    assert np.isfinite(o).all()
    assert attn_errors(o, ref).max() <= attn_tol(cfg), name


def test_attention_custom_scale_and_determinism():
    cfg = SMALL_ATTN["bf16_gqa_k8"]
    w = W.make_workload(cfg, sub_seed=3)
    t = to_device(w, DEV)
    o1 = run_attn(w, t, scale=0.05)
    o2 = run_attn(w, t, scale=0.05)
    assert np.array_equal(o1, o2)
    ref = R.verify_attn(w.q, w.k_cache, w.v_cache, w.kv_start, w.kv_len, w.k_new, w.v_new,
                        cfg.B, cfg.K, cfg.Hq, cfg.Hkv, cfg.D, scale=0.05)
    assert attn_errors(o1, ref).max() <= 1e-2


@pytest.mark.parametrize("name", ["bf16_gqa_k8", "fp32_d64_prefix"])
def test_attention_timing_events(name):
    """With dispatch-stamped timing events on, the result is unchanged and the
    events measure a positive duration."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    cfg = SMALL_ATTN[name]
    w = W.make_workload(cfg, sub_seed=5)
    t = to_device(w, DEV)
    o1 = run_attn(w, t)
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        api.sv_set_kernel_events(ev[0].value, ev[1].value)
        try:
            o2 = run_attn(w, t)
        finally:
            api.sv_set_kernel_events(None, None)
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value < 1000.0
    finally:
        for e in ev:
            hip.hipEventDestroy(e)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("heads", [(2, 2), (8, 2)])
def test_attention_device_lengths_against_host_bound(heads):
    """kv_len_host only bounds the device lengths: a device length above its
    sequence's bound (others unchanged) or a negative one sets status 3 and
    leaves that sequence unread; a device length below the bound gives the
    oracle's result for the device length.  With 8/2 heads and K = 8 the
    grouped-head kernel runs, whose even split then meets pieces with no key
    on the device."""
    Hq, Hkv = heads
    base = W.CONFIGS["bass_b8k5"] if Hq == Hkv else W.CONFIGS["gqa_b64k8"]
    cfg = W.small_variant(base, len_kind="uniform", B=4, Hq=Hq, Hkv=Hkv, len_lo=100, len_hi=300,
                          V=64)
    w = W.make_workload(cfg, sub_seed=12)
    t = to_device(w, DEV)
    for bad in (int(w.kv_len[1]) + 40, -1):
        kl = t.kv_len.clone()
        kl[1] = bad
        t.status.zero_()
        api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start, kl, w.kv_len, t.k_new,
                             t.v_new, t.out, cfg.K, status=t.status)
        torch.cuda.synchronize()
        assert int(t.status.item()) == 3, bad
    short = w.kv_len.copy()
    short[2] = max(0, int(short[2]) - 37)
    short[0] = 0
    t.status.zero_()
    api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start,
                         torch.from_numpy(short).to(DEV), w.kv_len, t.k_new, t.v_new, t.out,
                         cfg.K, status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0
    o = t.out.float().cpu().numpy().astype(np.float64)
    ref = R.verify_attn(w.q, w.k_cache, w.v_cache, w.kv_start, short, w.k_new, w.v_new, cfg.B,
                        cfg.K, cfg.Hq, cfg.Hkv, cfg.D)
    assert attn_errors(o, ref).max() <= 1e-2


def test_attention_bifurcated_equals_concatenated_gpu():
    """Prefix read once == the same prefix copied into every sequence's cache."""
    cfg = SMALL_ATTN["bf16_prefix"]
    w = W.make_workload(cfg, sub_seed=8)
    t = to_device(w, DEV)
    o_bif = run_attn(w, t)
    P = w.prefix_len
    lens = w.kv_len.astype(np.int64) + P
    caps = lens + cfg.K + 1
    starts = np.concatenate([[0], np.cumsum(caps)[:-1]])
    kc = np.zeros((int(caps.sum()), cfg.Hkv, cfg.D), np.uint16)
    vc = np.zeros_like(kc)
    for b in range(cfg.B):
        s, L = int(w.kv_start[b]), int(w.kv_len[b])
        kc[starts[b]:starts[b] + P] = w.k_prefix
        vc[starts[b]:starts[b] + P] = w.v_prefix
        kc[starts[b] + P:starts[b] + P + L] = w.k_cache[s:s + L]
        vc[starts[b] + P:starts[b] + P + L] = w.v_cache[s:s + L]
    out = torch.empty_like(t.q)
    api.spec_verify_attn(t.q, kv_tensor(kc, DEV), kv_tensor(vc, DEV),
                         torch.from_numpy(starts.astype(np.int64)).to(DEV),
                         torch.from_numpy(lens.astype(np.int32)).to(DEV), lens, t.k_new,
                         t.v_new, out, cfg.K)
    torch.cuda.synchronize()
    o_cat = out.float().cpu().numpy().astype(np.float64)
    ref = R.workload_attn(w)
    assert attn_errors(o_bif, ref).max() <= 1e-2
    assert attn_errors(o_cat, ref).max() <= 1e-2
    assert attn_errors(o_bif, o_cat).max() <= 1e-2


# ---------------------------------------------------------------- attention: full sizes

FULL = ["bass_b8k5", "chinchilla_b1k4", "gqa_b64k8", "prefix_b32k4"]


def oracle_attn_threaded(w, pairs):
    """Oracle attention of the listed (row, head) pairs, split over host threads
    (each thread calls the single-threaded oracle on its share; the foreign call
    releases the interpreter lock).  Returns [len(pairs), D] float64."""
    import concurrent.futures as cf
    import os as _os
    rows = np.asarray([r for r, _ in pairs], np.int32)
    heads = np.asarray([h for _, h in pairs], np.int32)
    n = rows.shape[0]
    nthr = max(1, min(16, _os.cpu_count() or 1))
    step = max(1, (n + 4 * nthr - 1) // (4 * nthr))
    parts = [(i, min(n, i + step)) for i in range(0, n, step)]
    out = np.zeros((n, w.cfg.D), np.float64)
    with cf.ThreadPoolExecutor(nthr) as ex:
        futs = {ex.submit(R.workload_attn, w, rows[a:b], heads[a:b]): (a, b) for a, b in parts}
        for fu in cf.as_completed(futs):
            a, b = futs[fu]
            out[a:b] = fu.result()
    return out


@pytest.mark.parametrize("name", FULL)
def test_attention_full_size_all_rows(name):
    """Every output (row, head) of the full-size workload against the oracle,
    in the launch configuration the benchmark times."""
    cfg = W.CONFIGS[name]
    say(f"[attn full] {name}: generating")
    w = W.make_workload(cfg, sub_seed=0)
    t = to_device(w, DEV)
    say(f"[attn full] {name}: running B={cfg.B} K={cfg.K} Hq={cfg.Hq} Hkv={cfg.Hkv}")
    o = run_attn(w, t)
    assert np.isfinite(o).all()
    R_ = cfg.rows
    pairs = [(r, h) for r in range(R_) for h in range(cfg.Hq)]
    say(f"[attn full] {name}: oracle over {len(pairs)} (row, head) pairs")
    ref = oracle_attn_threaded(w, pairs).reshape(R_, cfg.Hq, cfg.D)
    err = attn_errors(o, ref)
    say(f"[attn full] {name}: max row error {float(err.max()):.3e}")
    assert err.max() <= 1e-2, (name, float(err.max()), np.unravel_index(np.argmax(err), err.shape))


# ---------------------------------------------------------------- sampler

ACCEPT_CFGS = ["tiny_fp32", "bass_b8k5", "chinchilla_b1k4", "chinchilla_b1k4_greedy",
               "gqa_b64k8", "prefix_b32k4"]


@pytest.mark.parametrize("name", ACCEPT_CFGS)
def test_accept_full_size(name):
    cfg = W.CONFIGS[name]
    budget = FlagBudget()
    seeds = range(6) if cfg.B * cfg.V < 2_000_000 else range(2)
    for sub in seeds:
        say(f"[accept] {name} seed {sub}")
        w = W.make_workload(cfg, sub_seed=sub, with_kv=False)
        t = to_device(w, DEV)
        n, toks = run_accept(w, t)
        ref = R.workload_accept(w)
        budget.add(ref)
        compare_accept(n, toks, ref, cfg.K, rows_of(w))
        pins.check_counts({"n_accepted": n, "out_tokens": toks}, w.draft_tokens, cfg.K, cfg.V)
    budget.check()


@pytest.mark.parametrize("logits", ["f32", "bf16"])
def test_accept_many_sequences_small_vocab(logits):
    """Ragged vocab (not a multiple of 4), many sequences, K=3, nucleus."""
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=512, K=3, V=1001, top_p=0.9, temperature=0.7)
    w = W.make_workload(cfg, sub_seed=4, with_kv=False)
    if logits == "bf16":
        # bf16 logits: the oracle sees the same (exactly upcast) values
        w.target_logits = W.bf16_bits_to_f32(W.f32_to_bf16_bits(w.target_logits))
        w.draft_logits = W.bf16_bits_to_f32(W.f32_to_bf16_bits(w.draft_logits))
    t = to_device(w, DEV, logits_dtype=torch.bfloat16 if logits == "bf16" else torch.float32)
    n, toks = run_accept(w, t)
    ref = R.workload_accept(w)
    compare_accept(n, toks, ref, cfg.K, rows_of(w))


def test_accept_draw_zero_weight_cases():
    """The hand-derived rounds of the oracle's draw pin, on the GPU: ids of zero
    weight are never drawn (u = 0 included)."""
    def sampler(zt, zd, tok, ua, us, T, top_p, greedy, top_k=0):
        return gpu_sampler(zt, zd, tok, ua, us, T, top_p, greedy, top_k)
    pins.check_draw_cases(sampler, os.path.join(os.path.dirname(__file__), "golden"))


def test_accept_k0_bonus_only():
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=64, K=0, V=5000)
    w = W.make_workload(cfg, sub_seed=2, with_kv=False)
    t = to_device(w, DEV)
    n, toks = run_accept(w, t)
    ref = R.workload_accept(w)
    compare_accept(n, toks, ref, 0, rows_of(w))
    assert np.all(n == 0)


def test_accept_p_equals_q_accepts_all():
    cfg = W.CONFIGS["bass_b8k5"]
    w = W.make_workload(cfg, sub_seed=9, with_kv=False)
    w.draft_logits = np.ascontiguousarray(w.target_logits[:, : cfg.K])
    w.draft_tokens = np.argmax(w.draft_logits, axis=-1).astype(np.int32)
    t = to_device(w, DEV)
    n, toks = run_accept(w, t)
    assert np.all(n == cfg.K)
    compare_accept(n, toks, R.workload_accept(w), cfg.K, rows_of(w))


def test_accept_flat_rows_use_exact_fallback():
    """All-equal logits: the nucleus boundary bin holds the whole row (radix path)."""
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=4, K=2, V=8192, top_p=0.5)
    w = W.make_workload(cfg, sub_seed=1, with_kv=False)
    w.target_logits[:] = 0.25
    w.target_logits[1, 0, 17] = 3.0       # one peaked row mixed in
    w.draft_logits[:] = 0.25
    w.draft_tokens[:] = np.arange(cfg.B * cfg.K, dtype=np.int32).reshape(cfg.B, cfg.K) * 7
    t = to_device(w, DEV)
    n, toks = run_accept(w, t)
    compare_accept(n, toks, R.workload_accept(w), cfg.K, rows_of(w))


def test_accept_wide_rows_deep_threshold():
    """Low temperature and top_p close to 1: the nucleus boundary lies far below the max."""
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=16, K=3, V=20000, top_p=0.9999,
                          temperature=0.05, target_sigma=1.0)
    w = W.make_workload(cfg, sub_seed=6, with_kv=False)
    t = to_device(w, DEV)
    n, toks = run_accept(w, t)
    compare_accept(n, toks, R.workload_accept(w), cfg.K, rows_of(w))


def test_accept_bad_token_sets_status():
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=4, K=2, V=3000)
    w = W.make_workload(cfg, sub_seed=1, with_kv=False)
    t = to_device(w, DEV)
    t.draft_tokens[2, 1] = cfg.V + 5
    api.spec_accept(t.target_logits, t.draft_logits, t.draft_tokens, t.u_accept, t.u_sample,
                    cfg.temperature, cfg.top_p, False, t.n_accepted, t.out_tokens,
                    status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 1


@pytest.mark.parametrize("case", ["dirichlet_v8", "nucleus", "temp_half", "disjoint", "topk2",
                                  "topk2_nucleus"])
def test_theorem1_on_gpu(case):
    """The GPU sampler passes the same Theorem-1 pins as the oracle (10^6 trials)."""
    c = {x.name: x for x in pins.make_cases()}[case]
    pv, res, tok = pins.theorem1_pvalues(gpu_sampler, c, seed=17)
    assert min(pv) > pins.ALPHA, pv
    assert all(abs(z) < 5 for z in pins.accept_rate_z(res, c))
    assert pins.scan_length_pvalue(res, c) > pins.ALPHA


@pytest.mark.parametrize("case", ["dirichlet_v8", "nucleus", "disjoint", "topk2_nucleus"])
def test_accept_gpu_matches_oracle_many_trials(case):
    """Same 200k trials through both: bit-exact outside flagged decisions."""
    c = {x.name: x for x in pins.make_cases()}[case]
    zt, zd, tok, ua, us = pins.make_trials(c, n=200_000, seed=3)
    res = gpu_sampler(zt, zd, tok, ua, us, c.temperature, c.top_p, False, top_k=c.top_k)
    ref = R.accept(zt, zd, tok, ua, us, c.temperature, c.top_p, top_k=c.top_k)
    compare_accept(res["n_accepted"], res["out_tokens"], ref, c.K,
                   (zt, zd, tok, c.temperature, c.top_p, c.top_k))


# ---------------------------------------------------------------- compaction

@pytest.mark.parametrize("name", ["tiny_fp32", "bass_b8k5", "bass_k0"])
def test_compaction_matches_oracle(name):
    """Sampler then compaction against the oracle; bass_k0 is plain decode
    (K = 0: the bonus token only, one appended row per sequence)."""
    if name == "tiny_fp32":
        cfg = W.CONFIGS[name]
    else:
        cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=8, Hq=4, Hkv=4, len_lo=5, len_hi=300,
                              V=4096, K=0 if name == "bass_k0" else 5)
    w = W.make_workload(cfg, sub_seed=12)
    t = to_device(w, DEV)
    n, toks = run_accept(w, t)
    t.status.zero_()
    api.spec_compact_kv(t.n_accepted, t.out_tokens, t.kv_len, t.kv_start, t.k_cache, t.v_cache,
                        t.k_new, t.v_new, t.tokens_packed, t.cu_tokens, status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0
    packed, cu, kl, kc, vc = R.compact_kv(n, toks, w.kv_len, w.kv_start, w.k_cache, w.v_cache,
                                          w.k_new, w.v_new, cfg.K, cfg.Hkv, cfg.D)
    assert np.array_equal(t.cu_tokens.cpu().numpy(), cu)
    assert np.array_equal(t.kv_len.cpu().numpy(), kl)
    assert np.array_equal(t.tokens_packed.cpu().numpy()[: cu[-1]], packed[: cu[-1]])
    view = np.uint16 if cfg.kv_dtype == W.BF16 else np.uint32
    got_k = t.k_cache.view(torch.int16 if view == np.uint16 else torch.int32).cpu().numpy()
    got_v = t.v_cache.view(torch.int16 if view == np.uint16 else torch.int32).cpu().numpy()
    assert np.array_equal(got_k.view(view), kc.view(view))
    assert np.array_equal(got_v.view(view), vc.view(view))


def test_two_stream_pipeline_matches_one_stream():
    """The pipelined schedule of the benchmark's overlap mode (batch i's sampler
    and compaction on a second stream while batch i+1's attention runs, a
    batch's next attention after its previous compaction), captured into a HIP
    graph, gives bit-identical attention outputs, tokens, packed tokens, KV
    lengths and caches to the same steps on one stream, and both agree with
    the oracle run through the same schedule."""
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=6, Hq=8, Hkv=8, len_lo=20, len_hi=700,
                          V=8192, K=4)
    S, steps = 3, 9
    growth = (cfg.K + 1) * (steps // S + 2)
    works = [W.make_workload(cfg, sub_seed=20 + s, growth_rows=growth) for s in range(S)]
    bounds = [[int(x) + growth for x in w.kv_len] for w in works]

    def run(two_streams):
        ds = [to_device(w, DEV) for w in works]
        wa = torch.zeros(max(api.spec_verify_attn_workspace_size(cfg.B, cfg.K, cfg.Hq, cfg.Hkv, cfg.D,
                                                                 api.SV_BF16, bnd, 0)
                             for bnd in bounds), dtype=torch.uint8, device=DEV)
        wacc = torch.zeros(api.spec_accept_workspace_size(cfg.B, cfg.K, cfg.V), dtype=torch.uint8,
                           device=DEV)
        outs = torch.zeros((steps,) + tuple(ds[0].out.shape), dtype=ds[0].out.dtype, device=DEV)
        sA, sB = torch.cuda.Stream(), torch.cuda.Stream()

        def attn(i):
            t = ds[i % S]
            api.spec_verify_attn(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, bounds[i % S],
                                 t.k_new, t.v_new, t.out, cfg.K, status=t.status, workspace=wa)
            outs[i].copy_(t.out)

        def rest(i):
            t = ds[i % S]
            api.spec_accept(t.target_logits, t.draft_logits, t.draft_tokens, t.u_accept, t.u_sample,
                            cfg.temperature, cfg.top_p, False, t.n_accepted, t.out_tokens,
                            status=t.status, workspace=wacc)
            api.spec_compact_kv(t.n_accepted, t.out_tokens, t.kv_len, t.kv_start, t.k_cache,
                                t.v_cache, t.k_new, t.v_new, t.tokens_packed, t.cu_tokens,
                                status=t.status)

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=sA):
            if two_streams:
                sB.wait_stream(sA)
                done = [None] * S
                for i in range(steps):
                    if done[i % S] is not None:
                        sA.wait_event(done[i % S])
                    attn(i)
                    ea = torch.cuda.Event()
                    ea.record(sA)
                    with torch.cuda.stream(sB):
                        sB.wait_event(ea)
                        rest(i)
                        ed = torch.cuda.Event()
                        ed.record(sB)
                    done[i % S] = ed
                sA.wait_stream(sB)
            else:
                for i in range(steps):
                    attn(i)
                    rest(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in ds:
            assert int(t.status.item()) == 0
        return outs.cpu(), [(t.n_accepted.cpu(), t.out_tokens.cpu(), t.tokens_packed.cpu(),
                             t.cu_tokens.cpu(), t.kv_len.cpu(), t.k_cache.cpu(), t.v_cache.cpu())
                            for t in ds]

    o1, r1 = run(False)
    o2, r2 = run(True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for a, b in zip(r1, r2):
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    # each batch advanced by its emitted tokens once per use
    for s, w in enumerate(works):
        uses = sum(1 for i in range(steps) if i % S == s)
        n = r1[s][0].numpy().astype(np.int64)
        assert np.array_equal(r1[s][4].numpy(), w.kv_len + uses * (n + 1))
    # The oracle runs the same schedule on the host: every step's attention
    # over the cache state its batch has reached, the sampler's tokens, and the
    # compaction of the GPU's tokens into that state; the pipelined run's final
    # states (bit-identical to the one-stream run above) must equal it.
    state = [(w.kv_len.copy(), w.k_cache.copy(), w.v_cache.copy()) for w in works]
    last = [None] * S
    for i in range(steps):
        s = i % S
        w = works[s]
        kl, kc, vc = state[s]
        say(f"[two streams] oracle step {i} (batch {s})")
        ref_o = R.verify_attn(w.q, kc, vc, w.kv_start, kl, w.k_new, w.v_new, cfg.B, cfg.K, cfg.Hq,
                              cfg.Hkv, cfg.D)
        got_o = o2[i].float().numpy().astype(np.float64)
        assert attn_errors(got_o, ref_o).max() <= attn_tol(cfg), (i, s)
        n_gpu, toks_gpu = r2[s][0].numpy(), r2[s][1].numpy()
        ref = R.accept(w.target_logits, w.draft_logits, w.draft_tokens, w.u_accept, w.u_sample,
                       cfg.temperature, cfg.top_p)
        compare_accept(n_gpu, toks_gpu, ref, cfg.K, rows_of(w))
        packed, cu, kl2, kc2, vc2 = R.compact_kv(n_gpu, toks_gpu, kl, w.kv_start, kc, vc, w.k_new,
                                                 w.v_new, cfg.K, cfg.Hkv, cfg.D)
        state[s] = (kl2, kc2, vc2)
        last[s] = (packed, cu)
    for s in range(S):
        kl, kc, vc = state[s]
        packed, cu = last[s]
        assert np.array_equal(r2[s][4].numpy(), kl)
        assert np.array_equal(r2[s][3].numpy(), cu)
        assert np.array_equal(r2[s][2].numpy()[: cu[-1]], packed[: cu[-1]])
        assert np.array_equal(r2[s][5].view(torch.int16).numpy().view(np.uint16), kc.view(np.uint16))
        assert np.array_equal(r2[s][6].view(torch.int16).numpy().view(np.uint16), vc.view(np.uint16))


def test_compaction_rejects_bad_count():
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=3, Hq=2, Hkv=2, len_lo=5, len_hi=30, V=512)
    w = W.make_workload(cfg, sub_seed=1)
    t = to_device(w, DEV)
    t.n_accepted.copy_(torch.tensor([1, cfg.K + 3, 0], dtype=torch.int32))
    t.out_tokens.fill_(3)
    api.spec_compact_kv(t.n_accepted, t.out_tokens, t.kv_len, t.kv_start, t.k_cache, t.v_cache,
                        t.k_new, t.v_new, t.tokens_packed, t.cu_tokens, status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 4
    kl = t.kv_len.cpu().numpy()
    assert kl[1] == w.kv_len[1] and kl[0] == w.kv_len[0] + 2 and kl[2] == w.kv_len[2] + 1
    assert t.cu_tokens.cpu().numpy().tolist() == [0, 2, 2, 3]


# ---------------------------------------------------------------- ragged draft lengths K_b

RAGGED_ATTN = {
    "bf16_mha_ragged": W.small_variant(W.CONFIGS["bass_b8k5"], B=7, K=5, Hq=4, Hkv=4, len_lo=0,
                                       len_hi=700, V=64),
    "bf16_gqa_ragged": W.small_variant(W.CONFIGS["gqa_b64k8"], len_kind="uniform", B=9, K=7,
                                       Hq=8, Hkv=2, len_lo=10, len_hi=900, V=64),
    "bf16_d64_ragged": W.small_variant(W.CONFIGS["bass_b8k5"], B=5, K=6, Hq=6, Hkv=3, D=64,
                                       len_lo=1, len_hi=300, V=64),
    "bf16_prefix_ragged": W.small_variant(W.CONFIGS["prefix_b32k4"], B=6, K=4, Hq=4, Hkv=4,
                                          prefix_len=700, len_lo=0, len_hi=40, V=64),
    "fp32_prefix_ragged": W.small_variant(W.CONFIGS["prefix_b32k4"], kv_dtype=W.F32, B=4, K=4,
                                          Hq=4, Hkv=2, D=64, prefix_len=100, len_lo=0,
                                          len_hi=90, V=64),
}


def ragged_lengths(cfg, seed):
    kb = W.ragged_draft_lengths(cfg, seed)
    kb[0], kb[-1] = 0, cfg.K  # always one plain-decode sequence and one full one
    return kb


def run_attn_ragged(rw, t):
    w = rw.base
    t.status.zero_()
    api.spec_verify_attn_ragged(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len, w.kv_len,
                                t.k_new, t.v_new, t.out, t.cu_q, t.cu_q_host,
                                k_prefix=t.k_prefix, v_prefix=t.v_prefix, status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0
    return t.out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(RAGGED_ATTN))
def test_attention_ragged(name):
    cfg = RAGGED_ATTN[name]
    say(f"[attn ragged] {name}")
    rw = W.make_ragged(W.make_workload(cfg, sub_seed=2), ragged_lengths(cfg, 2))
    w = rw.base
    t = ragged_to_device(rw, DEV)
    o = run_attn_ragged(rw, t)
    ref = R.verify_attn_ragged(rw.q, w.k_cache, w.v_cache, w.kv_start, w.kv_len, rw.k_new,
                               rw.v_new, rw.cu_q, cfg.Hq, cfg.Hkv, cfg.D, k_prefix=w.k_prefix,
                               v_prefix=w.v_prefix)
    assert np.isfinite(o).all()
    err = attn_errors(o, ref)
    assert err.max() <= attn_tol(cfg), (name, float(err.max()))


@pytest.mark.parametrize("name", ["bf16_gqa_ragged", "fp32_prefix_ragged"])
def test_attention_ragged_equal_lengths_is_uniform(name):
    """cu_q[b] = b*(K+1): the ragged call gives the uniform call's bits."""
    cfg = RAGGED_ATTN[name]
    w = W.make_workload(cfg, sub_seed=4)
    rw = W.make_ragged(w, np.full(cfg.B, cfg.K, np.int32))
    o_r = run_attn_ragged(rw, ragged_to_device(rw, DEV))
    o_u = run_attn(w, to_device(w, DEV))
    assert np.array_equal(o_r, o_u)


def run_accept_ragged(rw, t, greedy):
    c = rw.cfg
    t.status.zero_()
    api.spec_accept_ragged(t.target_logits, None if greedy else t.draft_logits, t.draft_tokens,
                           t.u_accept, t.u_sample, t.cu_q, t.cu_q_host, c.temperature, c.top_p,
                           greedy, t.n_accepted, t.out_tokens, status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0, api.device_error_name(int(t.status.item()))
    return t.n_accepted.cpu().numpy(), t.out_tokens.cpu().numpy()


def compare_accept_ragged(n, toks, ref, cu, rows=None):
    """compare_accept for outputs packed by cu_q (b's tokens at cu[b] .. cu[b+1]-1);
    ``rows`` = (packed target logits, packed draft logits, packed drafts, T,
    top_p, top_k) enables the validity check of flagged sequences."""
    full = 0
    for b in range(n.shape[0]):
        f, nr = int(ref["flag_pos"][b]), int(ref["n_accepted"][b])
        got, exp = toks[cu[b]:cu[b + 1]], ref["out_tokens"][cu[b]:cu[b + 1]]
        if f < 0 or f > nr:
            assert n[b] == nr, (b, n[b], nr)
            assert np.array_equal(got, exp), (b, got, exp)
            full += 1
        else:
            assert n[b] >= f and np.array_equal(got[:f], exp[:f])
            if rows is not None:
                zt, zd, dr, T, tp, tk = rows
                k = int(cu[b + 1] - cu[b]) - 1
                d0 = int(cu[b]) - b
                check_flagged_valid(int(n[b]), got, zt[cu[b]:cu[b + 1]],
                                    None if zd is None else zd[d0:d0 + k], dr[d0:d0 + k], T,
                                    tp, tk)
    return full


@pytest.mark.parametrize("case", ["nucleus", "no_nucleus", "greedy", "bf16_logits"])
def test_accept_ragged(case):
    base = W.small_variant(W.CONFIGS["bass_b8k5"], B=40, K=7, V=9000)
    if case == "no_nucleus":
        base = W.small_variant(base, top_p=1.0, temperature=1.3)
    if case == "greedy":
        base = W.small_variant(base, greedy=True)
    budget = FlagBudget()
    full = 0
    for seed in range(3):
        say(f"[accept ragged] {case} seed {seed}")
        w = W.make_workload(base, sub_seed=seed, with_kv=False)
        if case == "bf16_logits":  # logits exactly representable in bf16
            w.target_logits = W.bf16_bits_to_f32(W.f32_to_bf16_bits(w.target_logits))
            w.draft_logits = W.bf16_bits_to_f32(W.f32_to_bf16_bits(w.draft_logits))
        rw = W.make_ragged(w, ragged_lengths(base, seed))
        t = ragged_to_device(rw, DEV, logits_dtype=torch.bfloat16 if case == "bf16_logits"
                             else torch.float32)
        n, toks = run_accept_ragged(rw, t, base.greedy)
        ref = R.accept_ragged(rw.target_logits, None if base.greedy else rw.draft_logits,
                              rw.draft_tokens, rw.u_accept, w.u_sample, rw.cu_q,
                              base.temperature, base.top_p, base.greedy)
        budget.add(ref)
        full += compare_accept_ragged(
            n, toks, ref, rw.cu_q,
            (rw.target_logits, None if base.greedy else rw.draft_logits, rw.draft_tokens,
             base.temperature, base.top_p, 0))
        assert np.all(n >= 0) and np.all(n <= rw.kb)
    budget.check()
    assert full >= 3 * base.B - 2


def test_compaction_ragged():
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=9, K=6, Hq=4, Hkv=4, len_lo=5, len_hi=300,
                          V=4096)
    rw = W.make_ragged(W.make_workload(cfg, sub_seed=8), ragged_lengths(cfg, 8))
    w = rw.base
    t = ragged_to_device(rw, DEV)
    n, toks = run_accept_ragged(rw, t, False)
    t.status.zero_()
    api.spec_compact_kv_ragged(t.n_accepted, t.out_tokens, t.kv_len, t.kv_start, t.k_cache,
                               t.v_cache, t.k_new, t.v_new, t.tokens_packed, t.cu_tokens, t.cu_q,
                               status=t.status)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0
    packed, cu, kl, kc, vc = R.compact_kv_ragged(n, toks, w.kv_len, w.kv_start, w.k_cache,
                                                 w.v_cache, rw.k_new, rw.v_new, rw.cu_q,
                                                 cfg.Hkv, cfg.D)
    assert np.array_equal(t.cu_tokens.cpu().numpy(), cu)
    assert np.array_equal(t.kv_len.cpu().numpy(), kl)
    assert np.array_equal(t.tokens_packed.cpu().numpy()[: cu[-1]], packed[: cu[-1]])
    assert np.array_equal(t.k_cache.view(torch.int16).cpu().numpy().view(np.uint16),
                          kc.view(np.uint16))
    assert np.array_equal(t.v_cache.view(torch.int16).cpu().numpy().view(np.uint16),
                          vc.view(np.uint16))


def test_workspace_reuse_across_lengths_and_draft_counts():
    """One zeroed workspace per entry point serves calls whose KV lengths and
    draft lengths differ (same B): every result equals that of a fresh
    workspace (attention) or the oracle (sampler)."""
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=6, K=5, Hq=4, Hkv=4, len_lo=0, len_hi=1500,
                          V=6000)
    rws = [W.make_ragged(W.make_workload(cfg, sub_seed=30 + s), ragged_lengths(cfg, 30 + s))
           for s in range(4)]
    ts = [ragged_to_device(rw, DEV) for rw in rws]
    wa = torch.zeros(max(api.spec_verify_attn_ragged_workspace_size(
        cfg.B, cfg.Hq, cfg.Hkv, cfg.D, api.SV_BF16, rw.base.kv_len, rw.cu_q) for rw in rws),
        dtype=torch.uint8, device=DEV)
    wacc = torch.zeros(max(api.spec_accept_ragged_workspace_size(cfg.B, rw.cu_q, cfg.V)
                           for rw in rws), dtype=torch.uint8, device=DEV)
    fresh = [run_attn_ragged(rw, t) for rw, t in zip(rws, ts)]
    for rep in range(2):
        for s, (rw, t) in enumerate(zip(rws, ts)):
            say(f"[workspace reuse] rep {rep} set {s} K_b {rw.kb.tolist()}")
            t.status.zero_()
            t.out.zero_()
            api.spec_verify_attn_ragged(t.q, t.k_cache, t.v_cache, t.kv_start, t.kv_len,
                                        rw.base.kv_len, t.k_new, t.v_new, t.out, t.cu_q,
                                        t.cu_q_host, status=t.status, workspace=wa)
            t.n_accepted.fill_(-7)
            api.spec_accept_ragged(t.target_logits, t.draft_logits, t.draft_tokens, t.u_accept,
                                   t.u_sample, t.cu_q, t.cu_q_host, cfg.temperature, cfg.top_p,
                                   False, t.n_accepted, t.out_tokens, status=t.status,
                                   workspace=wacc)
            torch.cuda.synchronize()
            assert int(t.status.item()) == 0
            o = t.out.float().cpu().numpy().astype(np.float64)
            assert np.array_equal(o, fresh[s])
            ref = R.accept_ragged(rw.target_logits, rw.draft_logits, rw.draft_tokens,
                                  rw.u_accept, rw.base.u_sample, rw.cu_q, cfg.temperature,
                                  cfg.top_p)
            compare_accept_ragged(t.n_accepted.cpu().numpy(), t.out_tokens.cpu().numpy(), ref,
                                  rw.cu_q, (rw.target_logits, rw.draft_logits, rw.draft_tokens,
                                            cfg.temperature, cfg.top_p, 0))



# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("top_k,top_p", [(1, 1.0), (20, 1.0), (300, 1.0), (20, 0.95), (300, 0.9),
                                         (5000, 1.0), (5000, 0.95), (8999, 0.95)])
def test_accept_topk(top_k, top_p):
    """Top-k (then nucleus) against the oracle.  k = 1 is the greedy rule; k =
    5000 of V = 9000 is beyond the candidate lists (radix select path)."""
    base = W.small_variant(W.CONFIGS["bass_b8k5"], B=24, K=5, V=9000, top_p=top_p)
    budget = FlagBudget()
    full = 0
    for seed in range(2):
        say(f"[accept topk] k={top_k} top_p={top_p} seed {seed}")
        w = W.make_workload(base, sub_seed=seed, with_kv=False)
        t = to_device(w, DEV)
        t.status.zero_()
        api.spec_accept(t.target_logits, t.draft_logits, t.draft_tokens, t.u_accept, t.u_sample,
                        base.temperature, base.top_p, False, t.n_accepted, t.out_tokens,
                        status=t.status, top_k=top_k)
        torch.cuda.synchronize()
        assert int(t.status.item()) == 0
        ref = R.accept(w.target_logits, w.draft_logits, w.draft_tokens, w.u_accept, w.u_sample,
                       base.temperature, base.top_p, top_k=top_k)
        budget.add(ref)
        full += compare_accept(t.n_accepted.cpu().numpy(), t.out_tokens.cpu().numpy(), ref,
                               base.K, rows_of(w, top_k))
    budget.check()
    assert full >= 2 * base.B - 2


@pytest.mark.parametrize("V,top_k,top_p", [(65536, 0, 0.95), (50001, 0, 0.95), (61441, 40, 0.95),
                                           (57344, 300, 1.0)])
def test_accept_list_path_segment_counts(V, top_k, top_p):
    """The candidate-list path at 13 to 16 segments of 4096 logits per row (its
    upper end), with a vocabulary that is not a multiple of 4 (scalar loads),
    nucleus and top-k, on the B=8, K=5 workload's logit distributions."""
    base = W.small_variant(W.CONFIGS["bass_b8k5"], V=V, top_p=top_p)
    budget = FlagBudget()
    full = 0
    for seed in range(2):
        say(f"[accept lists] V={V} top_k={top_k} top_p={top_p} seed {seed}")
        w = W.make_workload(base, sub_seed=seed, with_kv=False)
        t = to_device(w, DEV)
        t.status.zero_()
        api.spec_accept(t.target_logits, t.draft_logits, t.draft_tokens, t.u_accept, t.u_sample,
                        base.temperature, base.top_p, False, t.n_accepted, t.out_tokens,
                        status=t.status, top_k=top_k)
        torch.cuda.synchronize()
        assert int(t.status.item()) == 0
        ref = R.accept(w.target_logits, w.draft_logits, w.draft_tokens, w.u_accept, w.u_sample,
                       base.temperature, base.top_p, top_k=top_k)
        budget.add(ref)
        full += compare_accept(t.n_accepted.cpu().numpy(), t.out_tokens.cpu().numpy(), ref,
                               base.K, rows_of(w, top_k))
    budget.check()
    assert full >= 2 * base.B - 2


def test_accept_topk_ragged():
    base = W.small_variant(W.CONFIGS["bass_b8k5"], B=30, K=6, V=7000, top_p=0.9)
    for seed in range(2):
        w = W.make_workload(base, sub_seed=40 + seed, with_kv=False)
        rw = W.make_ragged(w, ragged_lengths(base, 40 + seed))
        t = ragged_to_device(rw, DEV)
        t.status.zero_()
        api.spec_accept_ragged(t.target_logits, t.draft_logits, t.draft_tokens, t.u_accept,
                               t.u_sample, t.cu_q, t.cu_q_host, base.temperature, base.top_p,
                               False, t.n_accepted, t.out_tokens, status=t.status, top_k=50)
        torch.cuda.synchronize()
        assert int(t.status.item()) == 0
        ref = R.accept_ragged(rw.target_logits, rw.draft_logits, rw.draft_tokens, rw.u_accept,
                              w.u_sample, rw.cu_q, base.temperature, base.top_p, top_k=50)
        compare_accept_ragged(t.n_accepted.cpu().numpy(), t.out_tokens.cpu().numpy(), ref,
                              rw.cu_q, (rw.target_logits, rw.draft_logits, rw.draft_tokens,
                                        base.temperature, base.top_p, 50))


# ---------------------------------------------------------------- maximum sizes

@pytest.mark.parametrize("top_k", [0, 100])
def test_accept_max_vocab_and_drafts(top_k):
    """V = 2^18 (64 segments: beyond the list path, radix select and whole-row
    draw) and K = 64 drafts (129 rows per sequence)."""
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=2, K=64, V=1 << 18, top_p=0.95)
    say(f"[accept max] top_k={top_k}")
    w = W.make_workload(cfg, sub_seed=9, with_kv=False)
    t = to_device(w, DEV)
    t.status.zero_()
    api.spec_accept(t.target_logits, t.draft_logits, t.draft_tokens, t.u_accept, t.u_sample,
                    cfg.temperature, cfg.top_p, False, t.n_accepted, t.out_tokens,
                    status=t.status, top_k=top_k)
    torch.cuda.synchronize()
    assert int(t.status.item()) == 0
    ref = R.accept(w.target_logits, w.draft_logits, w.draft_tokens, w.u_accept, w.u_sample,
                   cfg.temperature, cfg.top_p, top_k=top_k)
    compare_accept(t.n_accepted.cpu().numpy(), t.out_tokens.cpu().numpy(), ref, cfg.K,
                   rows_of(w, top_k))


def test_attention_max_sequences_and_columns():
    """B = 2048 sequences (the bf16 per-call limit) with short caches, and
    (Hq/Hkv)*(K+1) = 64 query columns per kv head (K = 63, MHA)."""
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=2048, K=1, Hq=2, Hkv=2, D=64, len_lo=0,
                          len_hi=12, V=64)
    w = W.make_workload(cfg, sub_seed=3)
    o = run_attn(w, to_device(w, DEV))
    assert attn_errors(o, R.workload_attn(w)).max() <= 1e-2
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], B=3, K=63, Hq=2, Hkv=2, len_lo=0,
                          len_hi=400, V=64)
    w = W.make_workload(cfg, sub_seed=4)
    o = run_attn(w, to_device(w, DEV))
    assert attn_errors(o, R.workload_attn(w)).max() <= 1e-2


# ---------------------------------------------------------------- fused compaction

def _fused_case(case):
    over = dict(B=8, Hq=4, Hkv=4, len_lo=5, len_hi=300, V=4096, K=5)
    top_k = 0
    if case == "greedy":
        over["greedy"] = True
    elif case == "no_filter":
        over["top_p"] = 1.0
    elif case == "k0":
        over["K"] = 0
    elif case == "topk":
        top_k = 20
    cfg = W.small_variant(W.CONFIGS["bass_b8k5"], **over)
    return cfg, top_k


@pytest.mark.parametrize("case", ["nucleus", "greedy", "no_filter", "topk", "k0", "ragged"])
def test_accept_compact_matches_two_calls_and_oracle(case):
    """spec_accept_compact equals spec_accept_ex followed by spec_compact_kv on
    the same inputs, bit for bit (tokens, counts, KV lengths, caches, packed
    tokens, offsets), over two rounds on one workspace (its counters must come
    back to zero); its tokens agree with the oracle and its compaction with the
    oracle's compaction of those tokens."""
    cfg, top_k = _fused_case("nucleus" if case == "ragged" else case)
    growth = 2 * (cfg.K + 1)
    w = W.make_workload(cfg, sub_seed=40, growth_rows=growth)
    ragged = case == "ragged"
    rw = W.make_ragged(w, ragged_lengths(cfg, 40)) if ragged else None
    say(f"[accept_compact] {case}")

    def dev():
        return ragged_to_device(rw, DEV) if ragged else to_device(w, DEV)

    g = cfg.greedy
    ta, tb = dev(), dev()
    if ragged:
        wsz = api.spec_accept_ragged_workspace_size(cfg.B, rw.cu_q, cfg.V)
    else:
        wsz = api.spec_accept_workspace_size(cfg.B, cfg.K, cfg.V)
    wa = torch.zeros(wsz, dtype=torch.uint8, device=DEV)
    wb = torch.zeros(wsz, dtype=torch.uint8, device=DEV)
    rounds = []
    for rnd in range(2):
        for t in (ta, tb):
            t.status.zero_()
        # two calls
        if ragged:
            api.spec_accept_ragged(ta.target_logits, None if g else ta.draft_logits, ta.draft_tokens,
                                   ta.u_accept, ta.u_sample, ta.cu_q, ta.cu_q_host, cfg.temperature,
                                   cfg.top_p, g, ta.n_accepted, ta.out_tokens, status=ta.status,
                                   workspace=wa, top_k=top_k)
            api.spec_compact_kv_ragged(ta.n_accepted, ta.out_tokens, ta.kv_len, ta.kv_start,
                                       ta.k_cache, ta.v_cache, ta.k_new, ta.v_new,
                                       ta.tokens_packed, ta.cu_tokens, ta.cu_q, status=ta.status)
        else:
            api.spec_accept(ta.target_logits, None if g else ta.draft_logits, ta.draft_tokens,
                            ta.u_accept, ta.u_sample, cfg.temperature, cfg.top_p, g,
                            ta.n_accepted, ta.out_tokens, status=ta.status, workspace=wa,
                            top_k=top_k)
            api.spec_compact_kv(ta.n_accepted, ta.out_tokens, ta.kv_len, ta.kv_start, ta.k_cache,
                                ta.v_cache, ta.k_new, ta.v_new, ta.tokens_packed, ta.cu_tokens,
                                status=ta.status)
        # one call
        api.spec_accept_compact(tb.target_logits, None if g else tb.draft_logits, tb.draft_tokens,
                                tb.u_accept, tb.u_sample, cfg.temperature, cfg.top_p, g,
                                tb.n_accepted, tb.out_tokens, tb.kv_len, tb.kv_start, tb.k_cache,
                                tb.v_cache, tb.k_new, tb.v_new, tb.tokens_packed, tb.cu_tokens,
                                status=tb.status, workspace=wb, top_k=top_k,
                                cu_q=tb.cu_q if ragged else None,
                                cu_q_host=tb.cu_q_host if ragged else None)
        torch.cuda.synchronize()
        assert int(ta.status.item()) == 0 and int(tb.status.item()) == 0
        for name in ("n_accepted", "out_tokens", "kv_len", "cu_tokens"):
            assert torch.equal(getattr(ta, name), getattr(tb, name)), (case, rnd, name)
        cu_end = int(tb.cu_tokens[-1].item())
        assert torch.equal(ta.tokens_packed[:cu_end], tb.tokens_packed[:cu_end]), (case, rnd)
        bits = torch.int16 if ta.k_cache.dtype == torch.bfloat16 else torch.int32  # spare rows hold NaN
        assert torch.equal(ta.k_cache.view(bits), tb.k_cache.view(bits)), (case, rnd)
        assert torch.equal(ta.v_cache.view(bits), tb.v_cache.view(bits)), (case, rnd)
        rounds.append((tb.n_accepted.cpu().numpy().copy(), tb.out_tokens.cpu().numpy().copy(),
                       tb.tokens_packed.cpu().numpy().copy(), tb.cu_tokens.cpu().numpy().copy(),
                       tb.kv_len.cpu().numpy().copy()))
    # the oracle: tokens (the same inputs both rounds) and the first round's compaction
    n, toks = rounds[0][0], rounds[0][1]
    if ragged:
        ref = R.accept_ragged(rw.target_logits, None if g else rw.draft_logits, rw.draft_tokens,
                              rw.u_accept, w.u_sample, rw.cu_q, cfg.temperature, cfg.top_p, g,
                              top_k=top_k)
        compare_accept_ragged(n, toks, ref, rw.cu_q,
                              (rw.target_logits, None if g else rw.draft_logits, rw.draft_tokens,
                               cfg.temperature, cfg.top_p, top_k))
        packed, cu, kl, _, _ = R.compact_kv_ragged(n, toks, w.kv_len, w.kv_start, w.k_cache,
                                                   w.v_cache, rw.k_new, rw.v_new, rw.cu_q,
                                                   cfg.Hkv, cfg.D)
    else:
        ref = R.accept(w.target_logits, None if g else w.draft_logits, w.draft_tokens, w.u_accept,
                       w.u_sample, cfg.temperature, cfg.top_p, g, top_k=top_k)
        compare_accept(n, toks, ref, cfg.K, rows_of(w, top_k))
        packed, cu, kl, _, _ = R.compact_kv(n, toks, w.kv_len, w.kv_start, w.k_cache, w.v_cache,
                                            w.k_new, w.v_new, cfg.K, cfg.Hkv, cfg.D)
    assert np.array_equal(rounds[0][3], cu)
    assert np.array_equal(rounds[0][2][: cu[-1]], packed[: cu[-1]])
    assert np.array_equal(rounds[0][4], kl)
    # the second round appended the same tokens' rows again
    e = (n.astype(np.int64) + 1)
    assert np.array_equal(rounds[1][4], kl + e)
