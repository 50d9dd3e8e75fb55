"""Seeded synthetic inputs for the batched speculative-sampling verify step.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests: both sides consume exactly the arrays it returns.  It holds no
arithmetic of the verify step itself (no attention, no softmax normaliser, no
accept test, no resample).  The only distribution it samples from is the
draft model's own decoding distribution, which the speculative-sampling paper
("Accelerating Large Language Model Decoding with Speculative Sampling",
section "Modified rejection sampling") places *before* verification: the K
draft tokens are draws from the draft model after its temperature/nucleus
modification.  That sampler is written here with a sort + Gumbel-max method,
which is a different algorithm from the inverse-CDF draw the verify step uses,
and the verify path never calls it.

Workload shapes follow the pages' workloads:
  * batch 8 with a 7.8B-class target (BASS abstract),
  * batch 1, K=4 on a 70B-class target with nucleus 0.8 / greedy
    (speculative-sampling paper, Table 1 and the XSum setup),
  * a large ragged GQA batch,
  * 32 samples sharing an >8k-token prompt (bifurcated-attention abstract),
  * a tiny fp32 round that the oracle checks exhaustively.
No dataset is used; the XSum and HumanEval workloads are stood in for by
random logits with the decoding parameters those experiments state.

Random streams are spawned from ``numpy.random.SeedSequence`` in a fixed
order, so every array is a pure function of (config, seed).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = 0
BF16 = 1

DTYPE_NAMES = {F32: "f32", BF16: "bf16"}

# Fill value for cache rows beyond a sequence's valid length: a bf16/f32 NaN.
# A kernel that reads outside [kv_start, kv_start + kv_len) poisons its output.
_NAN_BF16 = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    K: int
    Hq: int
    Hkv: int
    D: int
    V: int
    kv_dtype: int
    len_kind: str          # "fixed" | "uniform" | "loguniform"
    len_lo: int
    len_hi: int
    fixed_lens: tuple = ()
    prefix_len: int = 0
    temperature: float = 1.0
    top_p: float = 1.0
    greedy: bool = False
    target_sigma: float = 3.0
    draft_kind: str = "add"  # "add": draft = a*target + N(0, s^2); "indep": N(0, s^2)
    draft_a: float = 1.0
    draft_sigma: float = 1.0
    seed: int = 1000

    @property
    def rows(self) -> int:
        """Number of verify rows (queries per head): B*(K+1)."""
        return self.B * (self.K + 1)


CONFIGS = {
    # Tiny fp32 round: B=2, K=4, 2 heads x D16 MHA, KV lengths {5, 9}, V=32,
    # independent N(0, 2^2) target and draft logits, T=1, no nucleus.
    "tiny_fp32": Config(
        name="tiny_fp32", B=2, K=4, Hq=2, Hkv=2, D=16, V=32, kv_dtype=F32,
        len_kind="fixed", len_lo=5, len_hi=9, fixed_lens=(5, 9),
        temperature=1.0, top_p=1.0, target_sigma=2.0,
        draft_kind="indep", draft_sigma=2.0, seed=1001),
    # BASS-like 7.8B verify step: B=8, K=5, 32/32 heads x D128, L ~ U{512..2048},
    # V=49152, bf16 KV, fp32 logits, T=0.8, nucleus 0.95, draft = target + N(0,1).
    "bass_b8k5": Config(
        name="bass_b8k5", B=8, K=5, Hq=32, Hkv=32, D=128, V=49152, kv_dtype=BF16,
        len_kind="uniform", len_lo=512, len_hi=2048,
        temperature=0.8, top_p=0.95, target_sigma=3.0,
        draft_kind="add", draft_a=1.0, draft_sigma=1.0, seed=1002),
    # 70B-class B=1, K=4, 64 heads x D128, L=512, V=32000, nucleus 0.8, T=1.
    "chinchilla_b1k4": Config(
        name="chinchilla_b1k4", B=1, K=4, Hq=64, Hkv=64, D=128, V=32000, kv_dtype=BF16,
        len_kind="fixed", len_lo=512, len_hi=512, fixed_lens=(512,),
        temperature=1.0, top_p=0.8, target_sigma=3.0,
        draft_kind="add", draft_a=1.0, draft_sigma=2.0, seed=1003),
    # Same shape, greedy decoding (argmax drafts, argmax acceptance).
    "chinchilla_b1k4_greedy": Config(
        name="chinchilla_b1k4_greedy", B=1, K=4, Hq=64, Hkv=64, D=128, V=32000,
        kv_dtype=BF16, len_kind="fixed", len_lo=512, len_hi=512, fixed_lens=(512,),
        greedy=True, target_sigma=3.0, draft_kind="add", draft_a=1.0, draft_sigma=2.0,
        seed=1003),
    # Large ragged GQA batch: B=64, K=8, 32 q / 8 kv heads x D128,
    # L log-uniform in [1024, 8192], V=128256, draft = 0.7*target + N(0, 2^2), T=1.
    "gqa_b64k8": Config(
        name="gqa_b64k8", B=64, K=8, Hq=32, Hkv=8, D=128, V=128256, kv_dtype=BF16,
        len_kind="loguniform", len_lo=1024, len_hi=8192,
        temperature=1.0, top_p=1.0, target_sigma=3.0,
        draft_kind="add", draft_a=0.7, draft_sigma=2.0, seed=1004),
    # Shared-prefix multi-sample verify: B=32 samples share an 8192-token prefix,
    # per-sample decode KV ~ U{0..256}, K=4, 32 heads x D128 MHA, V=32000,
    # T=0.8, nucleus 0.95, draft = target + N(0, 1.5^2).
    "prefix_b32k4": Config(
        name="prefix_b32k4", B=32, K=4, Hq=32, Hkv=32, D=128, V=32000, kv_dtype=BF16,
        len_kind="uniform", len_lo=0, len_hi=256, prefix_len=8192,
        temperature=0.8, top_p=0.95, target_sigma=3.0,
        draft_kind="add", draft_a=1.0, draft_sigma=1.5, seed=1005),
}


def small_variant(cfg: Config, **over) -> Config:
    """A copy of ``cfg`` with some fields replaced (for reduced-size parity cases)."""
    return dataclasses.replace(cfg, **over)


@dataclasses.dataclass
class Workload:
    cfg: Config
    seed_path: tuple
    # attention (bf16 arrays hold raw bf16 bit patterns as uint16)
    q: np.ndarray            # [B*(K+1), Hq, D]
    k_cache: np.ndarray      # [rows, Hkv, D]
    v_cache: np.ndarray      # [rows, Hkv, D]
    kv_start: np.ndarray     # [B] int64: first cache row of sequence b
    kv_len: np.ndarray       # [B] int32: rows cached before this step
    kv_cap: np.ndarray       # [B] int64: rows reserved for sequence b
    k_new: np.ndarray        # [B*(K+1), Hkv, D]
    v_new: np.ndarray        # [B*(K+1), Hkv, D]
    k_prefix: Optional[np.ndarray]  # [P, Hkv, D] or None
    v_prefix: Optional[np.ndarray]
    # sampler
    target_logits: np.ndarray  # [B, K+1, V] float32
    draft_logits: np.ndarray   # [B, K, V] float32
    draft_tokens: np.ndarray   # [B, K] int32
    u_accept: np.ndarray       # [B, K] float32 in [0, 1)
    u_sample: np.ndarray       # [B] float32 in [0, 1)

    @property
    def prefix_len(self) -> int:
        return 0 if self.k_prefix is None else int(self.k_prefix.shape[0])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + rounding) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """Exact float32 uniforms on the 2^-24 grid in [0, 1): (uint32 >> 8) * 2^-24."""
    u = rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64) >> np.uint64(8)
    return (u.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _normal_kv(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == BF16 else x


def _lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.len_kind == "fixed":
        lens = np.array(cfg.fixed_lens, dtype=np.int64)
        assert lens.shape == (cfg.B,)
    elif cfg.len_kind == "uniform":
        lens = rng.integers(cfg.len_lo, cfg.len_hi + 1, size=cfg.B)
    elif cfg.len_kind == "loguniform":
        lo, hi = np.log(cfg.len_lo), np.log(cfg.len_hi)
        lens = np.floor(np.exp(rng.uniform(lo, hi, size=cfg.B))).astype(np.int64)
        lens = np.clip(lens, cfg.len_lo, cfg.len_hi)
    else:
        raise ValueError(cfg.len_kind)
    return lens.astype(np.int32)


def _draft_sample(z: np.ndarray, temperature: float, top_p: float, greedy: bool,
                  rng: np.random.Generator) -> int:
    """Sample one draft token the way the draft model would decode.

    Greedy: argmax (lowest id on ties).  Otherwise: tempered logits, optionally
    restricted to the smallest tie-closed top set with mass >= top_p (found by
    sorting), then a Gumbel-max draw inside that set.
    """
    if greedy:
        return int(np.argmax(z))
    x = z.astype(np.float64) / float(np.float32(temperature))
    keep = np.ones(z.shape[0], dtype=bool)
    if top_p < 1.0:
        order = np.argsort(-z, kind="stable")
        w = np.exp(x[order] - x[order[0]])
        cum = np.cumsum(w) / w.sum()
        k = int(np.searchsorted(cum, float(np.float32(top_p)), side="left"))
        k = min(k, z.shape[0] - 1)
        keep = z >= z[order[k]]
    g = -np.log(-np.log(rng.uniform(np.finfo(np.float64).tiny, 1.0, size=z.shape[0])))
    score = np.where(keep, x + g, -np.inf)
    return int(np.argmax(score))


def make_workload(cfg: Config, sub_seed: int = 0, growth_rows: int = 0,
                  lens: Optional[np.ndarray] = None, with_kv: bool = True) -> Workload:
    """Build the inputs of one verify step for ``cfg``.

    ``growth_rows`` reserves that many extra cache rows per sequence beyond
    L_b + K + 1, so that repeated compaction (which appends accepted rows) stays
    inside each sequence's region.  ``lens`` overrides the sampled KV lengths.
    ``with_kv=False`` skips the attention tensors (they become 1-row
    placeholders) for sampler-only use; the sampler inputs are unchanged.
    """
    ss = np.random.SeedSequence([cfg.seed, sub_seed])
    (s_len, s_q, s_kc, s_vc, s_kn, s_vn, s_pre, s_tl, s_dn, s_dt,
     s_ua, s_us) = ss.spawn(12)
    B, K, Hq, Hkv, D, V = cfg.B, cfg.K, cfg.Hq, cfg.Hkv, cfg.D, cfg.V
    R = B * (K + 1)

    kv_len = _lengths(cfg, np.random.default_rng(s_len)) if lens is None \
        else np.asarray(lens, dtype=np.int32)
    assert kv_len.shape == (B,)
    cap = kv_len.astype(np.int64) + (K + 1) + growth_rows
    kv_start = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    rows = int(cap.sum())

    if not with_kv:
        R, Hq, Hkv, D, rows = 1, 1, 1, 8, 1
        kv_len = np.zeros(B, np.int32)
        kv_start = np.zeros(B, np.int64)
    q = _normal_kv(np.random.default_rng(s_q), (R, Hq, D), cfg.kv_dtype)
    fill = _NAN_BF16 if cfg.kv_dtype == BF16 else np.float32(np.nan)
    kdt = np.uint16 if cfg.kv_dtype == BF16 else np.float32
    k_cache = np.full((rows, Hkv, D), fill, dtype=kdt)
    v_cache = np.full((rows, Hkv, D), fill, dtype=kdt)
    rk, rv = np.random.default_rng(s_kc), np.random.default_rng(s_vc)
    for b in range(B if with_kv else 0):
        n = int(kv_len[b])
        s0 = int(kv_start[b])
        if n:
            k_cache[s0:s0 + n] = _normal_kv(rk, (n, Hkv, D), cfg.kv_dtype)
            v_cache[s0:s0 + n] = _normal_kv(rv, (n, Hkv, D), cfg.kv_dtype)
    k_new = _normal_kv(np.random.default_rng(s_kn), (R, Hkv, D), cfg.kv_dtype)
    v_new = _normal_kv(np.random.default_rng(s_vn), (R, Hkv, D), cfg.kv_dtype)
    k_prefix = v_prefix = None
    if cfg.prefix_len and with_kv:
        rp = np.random.default_rng(s_pre)
        k_prefix = _normal_kv(rp, (cfg.prefix_len, Hkv, D), cfg.kv_dtype)
        v_prefix = _normal_kv(rp, (cfg.prefix_len, Hkv, D), cfg.kv_dtype)

    rt = np.random.default_rng(s_tl)
    target = (rt.standard_normal((B, K + 1, V), dtype=np.float32)
              * np.float32(cfg.target_sigma))
    rd = np.random.default_rng(s_dn)
    noise = rd.standard_normal((B, K, V), dtype=np.float32) * np.float32(cfg.draft_sigma)
    if cfg.draft_kind == "add":
        draft = np.float32(cfg.draft_a) * target[:, :K, :] + noise
    elif cfg.draft_kind == "indep":
        draft = noise
    else:
        raise ValueError(cfg.draft_kind)
    draft = np.ascontiguousarray(draft, dtype=np.float32)

    rs = np.random.default_rng(s_dt)
    draft_tokens = np.empty((B, K), dtype=np.int32)
    for b in range(B):
        for j in range(K):
            draft_tokens[b, j] = _draft_sample(draft[b, j], cfg.temperature, cfg.top_p,
                                               cfg.greedy, rs)
    u_accept = uniforms(np.random.default_rng(s_ua), (B, K))
    u_sample = uniforms(np.random.default_rng(s_us), (B,))
    return Workload(cfg=cfg, seed_path=(cfg.seed, sub_seed), q=q, k_cache=k_cache,
                    v_cache=v_cache, kv_start=kv_start, kv_len=kv_len, kv_cap=cap,
                    k_new=k_new, v_new=v_new, k_prefix=k_prefix, v_prefix=v_prefix,
                    target_logits=target, draft_logits=draft, draft_tokens=draft_tokens,
                    u_accept=u_accept, u_sample=u_sample)


@dataclasses.dataclass
class RaggedWorkload:
    """Sequence b carries its own draft length K_b <= K: the first K_b + 1 query
    rows, new K/V rows and target rows, and the first K_b drafts, draft rows
    and accept uniforms of sequence b of a uniform workload, packed back to
    back without padding (row offsets cu_q).  Caches, lengths, prefix and
    u_sample are the base workload's."""
    base: Workload
    kb: np.ndarray             # [B] int32 draft length of each sequence
    cu_q: np.ndarray           # [B+1] int32: rows of sequence b are cu_q[b] .. cu_q[b+1]-1
    q: np.ndarray              # [cu_q[B], Hq, D]
    k_new: np.ndarray          # [cu_q[B], Hkv, D]
    v_new: np.ndarray
    target_logits: np.ndarray  # [cu_q[B], V]
    draft_logits: np.ndarray   # [cu_q[B] - B, V]
    draft_tokens: np.ndarray   # [cu_q[B] - B]
    u_accept: np.ndarray       # [cu_q[B] - B]

    @property
    def cfg(self) -> Config:
        return self.base.cfg


def ragged_draft_lengths(cfg: Config, sub_seed: int = 0) -> np.ndarray:
    """Seeded draft lengths K_b, uniform on 0..K (their own seed stream)."""
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, sub_seed, 0x4B62]))
    return rng.integers(0, cfg.K + 1, size=cfg.B).astype(np.int32)


def make_ragged(w: Workload, kb) -> RaggedWorkload:
    c = w.cfg
    B, K, V = c.B, c.K, c.V
    kb = np.asarray(kb, dtype=np.int32)
    assert kb.shape == (B,) and np.all(kb >= 0) and np.all(kb <= K)
    cu = np.concatenate([[0], np.cumsum(kb.astype(np.int64) + 1)]).astype(np.int32)
    iq = np.concatenate([b * (K + 1) + np.arange(kb[b] + 1) for b in range(B)])
    idr = np.concatenate([b * K + np.arange(kb[b]) for b in range(B)]).astype(np.int64)
    return RaggedWorkload(
        base=w, kb=kb, cu_q=cu,
        q=np.ascontiguousarray(w.q[iq]) if w.q.shape[0] == B * (K + 1) else w.q,
        k_new=np.ascontiguousarray(w.k_new[iq]) if w.k_new.shape[0] == B * (K + 1) else w.k_new,
        v_new=np.ascontiguousarray(w.v_new[iq]) if w.v_new.shape[0] == B * (K + 1) else w.v_new,
        target_logits=np.ascontiguousarray(w.target_logits.reshape(B * (K + 1), V)[iq]),
        draft_logits=np.ascontiguousarray(w.draft_logits.reshape(B * K, V)[idr]),
        draft_tokens=np.ascontiguousarray(w.draft_tokens.reshape(B * K)[idr]),
        u_accept=np.ascontiguousarray(w.u_accept.reshape(B * K)[idr]))


def algorithmic_bytes(cfg: Config, kv_len: np.ndarray, prefix_len: int = 0) -> dict:
    """Bytes the verify step must move at least once, by part.

    Attention: every cached KV row of every sequence once, the shared prefix once,
    the new K/V rows, Q read and O written.  Sampler: every target and draft
    logit row read once (greedy: target rows only), plus the per-sequence vectors.
    Compaction: the accepted new K/V rows it appends are counted separately.
    """
    es = 2 if cfg.kv_dtype == BF16 else 4
    row_kv = cfg.Hkv * cfg.D * es * 2           # K and V for one token
    R = cfg.rows
    attn = (int(np.sum(kv_len)) + prefix_len) * row_kv + R * row_kv \
        + 2 * R * cfg.Hq * cfg.D * es
    logit_rows = cfg.B * (cfg.K + 1) + (0 if cfg.greedy else cfg.B * cfg.K)
    accept = logit_rows * cfg.V * 4 + cfg.B * cfg.K * 8 + cfg.B * 4 + cfg.B * (cfg.K + 2) * 4
    return {"attn": attn, "accept": accept}
