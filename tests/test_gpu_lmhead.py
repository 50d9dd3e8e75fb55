"""LM head with the sampler's row statistics (spec_lm_head_stats) and the
sampler that takes them (spec_accept_prestats), against the oracle.

"Accelerating Large Language Model Decoding with Speculative Sampling",
"Conditional scoring": the target call ends in the LM head; the sampler's
first need from each row is its max and normaliser.
"""
import numpy as np
import pytest
import torch

from oracle import specref as R
from speculative_decoding_verify_04_amd import api
from speculative_decoding_verify_04_amd import workloads as W

from test_gpu_parity import compare_accept, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def bf16_inputs(rows, H, V, seed, wscale=0.08):
    rng = np.random.default_rng(seed)
    h = W.f32_to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    w = W.f32_to_bf16_bits((wscale * rng.standard_normal((V, H))).astype(np.float32))
    return h, w


def to_bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def run_lm_head(h, w, T):
    rows, H = h.shape
    V = w.shape[0]
    P = api.spec_lm_head_parts(V)
    logits = torch.empty((rows, V), dtype=torch.float32, device=DEV)
    pm = torch.empty((rows, P), dtype=torch.float32, device=DEV)
    ps = torch.empty((rows, P), dtype=torch.float64, device=DEV)
    api.spec_lm_head_stats(to_bf16(h), to_bf16(w), T, logits, pm, ps)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), pm.cpu().numpy(), ps.cpu().numpy()


def combine_parts(pm, ps, T):
    """Row max and normaliser from the parts, in fp64 on the host."""
    m = pm.max(axis=1).astype(np.float64)
    scale = np.where(pm == -np.inf, 0.0, np.exp((pm.astype(np.float64) - m[:, None]) / T))
    return m, (ps * scale).sum(axis=1)


@pytest.mark.parametrize("rows,H,V", [(48, 512, 12288), (5, 96, 1000), (130, 64, 302),
                                      (16, 2048, 4096), (1, 32, 129),
                                      # 17 to 64 rows: 192-id tiles of 2, 3 or 4 row tiles
                                      (17, 96, 500), (40, 224, 2000), (64, 32, 193),
                                      # more than 64 rows: the LDS-staged tiles (192 rows x 256
                                      # ids): several row blocks, partial id tiles, every count
                                      # of 32-wide steps modulo the five stages, one step
                                      (200, 256, 2000), (576, 128, 1030), (65, 32, 129),
                                      (384, 160, 4096)])
def test_lm_head_logits_and_part_statistics(rows, H, V):
    """Logits within the fp32-accumulation bound of the fp64 oracle
    (2^-24 H sum|h w| per element); every part's max and fp64 sum, and the row
    statistics combined from the parts, against the oracle's statistics of the
    GPU's own logits (max exact, sums to 1e-13 / 1e-12)."""
    T = float(np.float32(0.8))  # the library receives the temperature as float32
    say(f"[lm head] rows {rows} H {H} V {V}")
    h, w = bf16_inputs(rows, H, V, seed=rows + H + V)
    z, pm, ps = run_lm_head(h, w, T)
    ref = R.lm_head(h, w)
    habs = W.f32_to_bf16_bits(np.abs(W.bf16_bits_to_f32(h)))
    wabs = W.f32_to_bf16_bits(np.abs(W.bf16_bits_to_f32(w)))
    bound = 2.0 ** -24 * H * R.lm_head(habs, wabs) + 1e-30
    assert np.all(np.abs(z.astype(np.float64) - ref) <= bound)
    P = api.spec_lm_head_parts(V)
    assert pm.shape == (rows, P) and P == (V + 63) // 64  # parts of 64 ids
    for i in range(P):
        part = np.ascontiguousarray(z[:, 64 * i:min(V, 64 * (i + 1))])
        m_ref, s_ref = R.row_stats(part, T)
        assert np.array_equal(pm[:, i].astype(np.float64), m_ref)
        assert np.allclose(ps[:, i], s_ref, rtol=1e-13, atol=0)
    m, S = combine_parts(pm, ps, T)
    m_ref, S_ref = R.row_stats(z, T)
    assert np.array_equal(m, m_ref)
    assert np.allclose(S, S_ref, rtol=1e-12, atol=0)


def gumbel_draws(logits, T, rng):
    """Draft tokens drawn from softmax(logits / T) (Gumbel-max)."""
    g = -np.log(-np.log(rng.random(logits.shape)))
    return np.argmax(logits.astype(np.float64) / T + g, axis=-1).astype(np.int32)


@pytest.mark.parametrize("top_p", [1.0, 0.9])
def test_accept_prestats_with_lm_head_logits(top_p):
    """Target and draft rows from two LM heads (two weight matrices, the draft
    rows' hidden states perturbed): spec_accept_prestats against the oracle on
    the same fp32 logits.  Without a filter the statistics replace the segment
    pass; with a nucleus they are not used and the result is bit-identical to
    spec_accept."""
    B, K, H, V = 8, 5, 256, 6000
    T = float(np.float32(0.9))
    say(f"[lm head + prestats] top_p {top_p}")
    rng = np.random.default_rng(int(top_p * 100))
    ht, wt = bf16_inputs(B * (K + 1), H, V, seed=11, wscale=0.15)
    hprev = W.bf16_bits_to_f32(ht).reshape(B, K + 1, H)[:, :K].reshape(B * K, H)
    hd = W.f32_to_bf16_bits(hprev + 0.3 * rng.standard_normal((B * K, H)).astype(np.float32))
    _, wd = bf16_inputs(1, H, V, seed=12, wscale=0.15)
    zt, pmt, pst = run_lm_head(ht, wt, T)
    zd, pmd, psd = run_lm_head(hd, wd, T)
    drafts = gumbel_draws(zd, T, rng).reshape(B, K)
    ua = W.uniforms(rng, (B, K))
    us = W.uniforms(rng, (B,))
    zt3, zd3 = zt.reshape(B, K + 1, V), zd.reshape(B, K, V)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    n = torch.zeros(B, dtype=torch.int32, device=DEV)
    toks = torch.zeros((B, K + 1), dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    api.spec_accept_prestats(dev(zt3), dev(zd3), dev(drafts), dev(ua), dev(us), T, top_p, False, n,
                             toks, dev(pmt), dev(pst), dev(pmd), dev(psd), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = R.accept(zt3, zd3, drafts, ua, us, T, top_p)
    compare_accept(n.cpu().numpy(), toks.cpu().numpy(), ref, K,
                   (zt3, zd3, drafts, T, top_p, 0))
    if top_p < 1.0:
        n2 = torch.zeros_like(n)
        t2 = torch.zeros_like(toks)
        api.spec_accept(dev(zt3), dev(zd3), dev(drafts), dev(ua), dev(us), T, top_p, False, n2, t2,
                        status=status)
        torch.cuda.synchronize()
        assert torch.equal(n, n2) and torch.equal(toks, t2)
