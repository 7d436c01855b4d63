"""Seeded synthetic inputs and the named workloads of the attention path.

Holds no attention arithmetic: it only names shapes and draws the random
tensors that both the oracle (``oracle/``) and the HIP library are fed.

Recipe (the same for every workload): ``torch.Generator('cpu')`` seeded with
``seed`` draws Q, K, V, dO in that order with ``torch.randn`` in float32
(i.i.d. N(0, 1)); bf16 workloads then round each to bfloat16 (round to
nearest even).  The oracle receives exactly these values upcast to float64,
so input rounding is never counted as kernel error.

Shapes follow the pages' own workloads:
  * tiny fp32 causal / full self-attention (a correctness case);
  * the batch-8 d_model x seq_len grid of the CS336 Triton benchmark
    (head count 16 and causal masking are this library's choice; the page
    states neither);
  * long-context (16K / 32K) GQA causal attention, the SpecForge setting;
  * the EAGLE3 TTT call at draft step t = 2 (keys/values of steps 0, 1, 2
    concatenated, Skv = 3 * Sq);
  * diffusion-transformer full self-attention and cross-attention with padded
    keys (1000 valid of 1024), the ggml playbook's real geometries;
  * windowed self-attention, the playbook's third geometry (its window is
    not given: a symmetric band of +-512 keys on the DiT shape), and a
    causal sliding window of 4096 keys on the long-context GQA shape;
  * a causal sequence behind a frozen KV prefix (the playbook's per-trainer
    checklist names a trainer with a frozen/trained KV prefix and no sizes:
    4096 prefix keys before the 16K long-context GQA shape, prefix frozen).
"""
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

FULL, CAUSAL, TTT, WINDOW = 0, 1, 2, 3
KIND_NAMES = {FULL: "full", CAUSAL: "causal", TTT: "ttt", WINDOW: "window"}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    kind: int
    dtype: str = "bf16"            # "bf16" or "f32"
    shift: int = 0
    kv_valid: Optional[tuple] = None   # per-batch valid key count, None = all
    scale: Optional[float] = None      # None -> 1/sqrt(D)
    window: Optional[tuple] = None     # WINDOW: (left, right)
    frozen: int = 0                    # keys below it are frozen (no dK/dV)

    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw):
        return replace(self, **kw)


def tiny_fp32(kind=CAUSAL):
    return Workload(f"tiny_fp32_{KIND_NAMES[kind]}", 1, 2, 2, 128, 128, 64,
                    kind, dtype="f32")


def grid(D, S):
    return Workload(f"grid_D{D}_S{S}", 8, 16, 16, S, S, D, CAUSAL)


def long_gqa(S=16384):
    return Workload(f"long_gqa_S{S}", 1, 32, 4, S, S, 128, CAUSAL)


def ttt(S=16384, step=2, shift=0):
    return Workload(f"ttt_S{S}_t{step}", 1, 32, 4, S, (step + 1) * S, 128,
                    TTT, shift=shift)


def dit_self():
    return Workload("dit_self_S8192", 2, 16, 16, 8192, 8192, 64, FULL)


def dit_cross():
    return Workload("dit_cross_S8192_kv1000of1024", 2, 16, 16, 8192, 1024, 64,
                    FULL, kv_valid=(1000, 1000))


def dit_window(w=512):
    return Workload(f"dit_window_S8192_w{w}", 2, 16, 16, 8192, 8192, 64, WINDOW, window=(w, w))


def swa_gqa(S=16384, w=4096):
    return Workload(f"swa_gqa_S{S}_w{w}", 1, 32, 4, S, S, 128, WINDOW, window=(w - 1, 0))


def prefix_gqa(S=16384, P=4096):
    # a causal sequence behind a frozen P-key prefix (the rectangular mask a
    # frozen KV prefix needs): CAUSAL with shift -P over P + S keys
    return Workload(f"prefix_gqa_S{S}_P{P}_frozen", 1, 32, 4, S, P + S, 128, CAUSAL, shift=-P, frozen=P)


HEADLINE = long_gqa(16384)


def all_workloads():
    ws = [tiny_fp32(CAUSAL), tiny_fp32(FULL)]
    ws += [grid(D, S) for D in (16, 32, 64) for S in (256, 1024, 4096)]
    ws += [long_gqa(16384), long_gqa(32768), ttt(16384, 2), dit_self(),
           dit_cross(), dit_window(), swa_gqa(), prefix_gqa()]
    return ws


def make_inputs(w: Workload, seed: int = 0, device="cpu"):
    """Q, K, V, dO as [B, H, S, D] tensors of the workload's dtype.

    Drawn on the CPU generator (so every device sees identical values), then
    moved to ``device``.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    shapes = [(w.B, w.Hq, w.Sq, w.D), (w.B, w.Hkv, w.Skv, w.D),
              (w.B, w.Hkv, w.Skv, w.D), (w.B, w.Hq, w.Sq, w.D)]
    out = []
    for shp in shapes:
        x = torch.randn(shp, generator=g, dtype=torch.float32)
        out.append(x.to(w.torch_dtype()).to(device))
    return tuple(out)


def kv_valid_tensor(w: Workload, device="cpu"):
    if w.kv_valid is None:
        return None
    return torch.tensor(list(w.kv_valid), dtype=torch.int32, device=device)


# ---- stress inputs for the forward's running-max refresh ---------------------
# Scores of N(0, 1) inputs stay within a few units of the first key tile's
# maximum, so a forward that keeps a lazy running max (refreshed only when a
# tile's sum of exp(score - max) grows large) never rescales accumulators that
# already hold values on them.  These recipes make some keys score far above
# the ones before them (the SpecForge page warns that unbounded inputs break
# naive references; here every value stays bounded and finite).
#   spike:   u a seeded random unit vector of R^D.  q_i = sqrt(D) u + 0.1 n_i;
#            k_j = 0.1 m_j, except for the keys listed in `spikes`, where
#            k_j = level * u + 0.1 m_j; so with the default scale 1/sqrt(D)
#            scores are about 0 and, on the spike keys, about `level`.
#            v_j = +1 + 0.5 w_j (every component), and -1 + 0.5 w_j on the
#            spike keys, so the output before and after a spike differ in
#            sign.  n, m, w and dO are i.i.d. N(0, 1).
#   peaky:   the standard recipe with Q multiplied by 4.
#   uniform: Q, K, V, dO i.i.d. U(-1, 1).
# One CPU generator seeded with `seed` draws, in order: u (spike only), Q, K,
# V, dO.

def make_stress_inputs(recipe, B, Hq, Hkv, Sq, Skv, D, seed=0, spikes=(), level=7.0,
                       dtype=torch.bfloat16):
    g = torch.Generator("cpu").manual_seed(seed)
    qs, ks = (B, Hq, Sq, D), (B, Hkv, Skv, D)
    f64 = torch.float64
    if recipe == "spike":
        u = torch.randn(D, generator=g, dtype=f64)
        u = u / u.norm()
        hot = torch.zeros(Skv, dtype=f64)
        hot[list(spikes)] = 1.0
        q = D ** 0.5 * u + 0.1 * torch.randn(qs, generator=g, dtype=f64)
        k = (level * hot)[:, None] * u + 0.1 * torch.randn(ks, generator=g, dtype=f64)
        v = (1.0 - 2.0 * hot)[:, None] + 0.5 * torch.randn(ks, generator=g, dtype=f64)
        do = torch.randn(qs, generator=g, dtype=f64)
    elif recipe == "peaky":
        q = 4.0 * torch.randn(qs, generator=g, dtype=f64)
        k, v = (torch.randn(ks, generator=g, dtype=f64) for _ in range(2))
        do = torch.randn(qs, generator=g, dtype=f64)
    elif recipe == "uniform":
        q, k, v, do = (2 * torch.rand(s, generator=g, dtype=f64) - 1 for s in (qs, ks, ks, qs))
    else:
        raise ValueError(f"unknown recipe {recipe}")
    return tuple(x.to(dtype) for x in (q, k, v, do))


def make_key_bias(B, Skv, seed=0, lo=-3.0, hi=3.0, neg_inf_frac=0.15, device="cpu"):
    """A per-batch key bias [B, Skv] float32: uniform in [lo, hi) with a
    fraction of the keys at -inf (dropped), key 0 always finite."""
    g = torch.Generator().manual_seed(seed)
    b = torch.rand(B, Skv, generator=g) * (hi - lo) + lo
    drop = torch.rand(B, Skv, generator=g) < neg_inf_frac
    drop[:, 0] = False
    b[drop] = float("-inf")
    return b.to(device)


# ---- soft-target log-softmax loss workloads ---------------------------------
# The (B, T, V) configurations of the SpecForge page's loss benchmark (section
# "In-place Gradient Calculation").  Recipe: a generator on ``device`` seeded
# with ``seed`` draws the logits, float32 N(0, 1) times ``logit_std`` (4: the
# page gives no distribution), then u ~ U(0, 1), and the soft targets are
# u**8 normalised over the vocabulary (a peaked distribution, made without
# the loss's own arithmetic).  The first ``prompt_frac`` of each sequence's
# positions have mask 0 (the prompt, which EAGLE3 masks out), the rest 1.

@dataclass(frozen=True)
class LossWorkload:
    name: str
    B: int
    T: int
    V: int
    logit_std: float = 4.0
    prompt_frac: float = 0.1

    @property
    def N(self):
        return self.B * self.T


def loss_workloads():
    return [LossWorkload(f"lsm_loss_B{B}_T{T}_V{V}", B, T, V)
            for B, T, V in ((1, 1024, 32000), (1, 4096, 32000), (1, 4096, 64000),
                            (1, 8192, 32000), (1, 8192, 64000), (1, 16384, 32000))]


LOSS_HEADLINE = loss_workloads()[-1]


def make_loss_inputs(w: LossWorkload, seed: int = 0, device="cpu"):
    """(logits [N, V], target [N, V], mask [N]), float32 on ``device``."""
    g = torch.Generator(device).manual_seed(seed)
    x = torch.randn(w.N, w.V, generator=g, device=device) * w.logit_std
    u = torch.rand(w.N, w.V, generator=g, device=device) ** 8
    t = u / u.sum(dim=1, keepdim=True)
    pos = torch.arange(w.T, device=device).repeat(w.B)
    mask = (pos >= int(w.prompt_frac * w.T)).to(torch.float32)
    return x, t, mask
