"""Seeded synthetic workloads for the joint sCM target.

This module only draws and rounds numbers.  It holds none of the method's
arithmetic (no noising, no fields, no attention), so both the HIP path and the
fp64 checker can consume the same inputs without sharing any computation.

Workload shapes follow TurboT2VA (arXiv 2608.24674): the high-resolution
deployment setting packs a 1024x1792, 121-frame clip into a video latent of
shape [1, 16, 128, 32, 56], i.e. 16*32*56 = 28,672 video tokens with 128
channels (robotworld.top deep read, section 6.4); the 512x768 training/eval
resolution gives 16*16*24 = 6,144 tokens under the same packing (section 7).
Audio and text sizes, the block width and the head layout are the synthetic
choices listed in ``CONFIGS``.

Weights use the nn.Linear convention ``[out_features, in_features]``:
    w_in_v [d, Cv], w_in_a [d, Ca], w_t [d, d], w_qkv [3d, d] (rows: q | k | v),
    w_out_v [Cv, d], w_out_a [Ca, d].
Latents are row-major [B, N_m, C_m]; text is [B, Nt, d]; the text mask is
uint8 [B, Nt] with 1 = valid prompt token.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict

import numpy as np

HALF_PI = math.pi / 2.0


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    Nv: int
    Na: int
    Nt: int
    Ntv: int                 # valid text tokens per sample (prefix) unless mask_mode says otherwise
    Cv: int
    Ca: int
    d: int
    H: int
    in_dtype: str            # "bf16" or "fp32": storage type of latents, text and weights
    beta: float = 1.0
    gamma: float = 1.0
    eps_scm: float = 1e-6
    w_v: float = 1.0
    w_a: float = 1.0
    t_mode: str = "uniform"  # "uniform": U(0.05, pi/2-0.05); "edges": half near 0, half near pi/2
    z0_scale_v: float = 1.0
    z0_scale_a: float = 1.0
    mask_mode: str = "prefix"  # "prefix" or "scatter" (valid positions spread over the sequence)
    index: int = 0           # seed offset: data 100+index, teacher 200+index, student 300+index
    # The joint DMD term and the stage-3 mix: guidance scales of the teacher
    # prediction per modality (3.0 video, 5.0 audio, and equal sCM/DMD weights
    # in the pages' training setup), the residual-scale normaliser's epsilon.
    # Parameterisation of the block: "x0" (it predicts x0 at TrigFlow inputs)
    # or "rf" (a rectified-flow velocity model behind the TrigFlow wrapper).
    param: str = "x0"
    # Precision of the primal logit path on the GPU: "bf16" (bf16 storage
    # between kernels) or "split" (hi + lo bf16 pairs for the noised latents,
    # token rows, Q and K; for inputs whose large logits make attention
    # sensitive to bf16 rounding).  The oracle is exact fp64 either way.
    precision: str = "bf16"
    cfg_v: float = 3.0
    cfg_a: float = 5.0
    eps_dmd: float = 1e-6
    lam_scm: float = 1.0
    lam_dmd: float = 1.0

    @property
    def dh(self) -> int:
        return self.d // self.H

    @property
    def Nq(self) -> int:
        return self.Nv + self.Na

    @property
    def N_all(self) -> int:
        return self.Nv + self.Na + self.Nt

    def replace(self, **kw) -> "Config":
        a = asdict(self)
        a.update(kw)
        return Config(**a)


# The five workloads.  "60% padded" text: valid = 256 - round(0.6*256) = 102.
CONFIGS = {
    "tiny": Config("tiny", B=1, Nv=64, Na=16, Nt=8, Ntv=8, Cv=128, Ca=64, d=256, H=4,
                   in_dtype="fp32", beta=1.0, gamma=0.5, eps_scm=1e-6, index=0),
    "small": Config("small", B=2, Nv=1536, Na=128, Nt=128, Ntv=64, Cv=128, Ca=64, d=1024, H=8,
                    in_dtype="bf16", beta=1.0, gamma=1.0, index=1),
    "standard": Config("standard", B=1, Nv=6144, Na=256, Nt=256, Ntv=102, Cv=128, Ca=64, d=2048,
                       H=16, in_dtype="bf16", beta=1.0, gamma=1.0, index=2),
    "high-res": Config("high-res", B=1, Nv=28672, Na=256, Nt=256, Ntv=102, Cv=128, Ca=64, d=2048,
                       H=16, in_dtype="bf16", beta=1.0, gamma=1.0, index=3),
    "stress": Config("stress", B=8, Nv=1536, Na=1024, Nt=128, Ntv=128, Cv=128, Ca=64, d=1024, H=8,
                     in_dtype="bf16", beta=2.0, gamma=0.25, w_v=1.0, w_a=4.0, t_mode="edges",
                     z0_scale_v=10.0, z0_scale_a=0.1, index=4, precision="split"),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returns float64 values."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def draw_t(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.t_mode == "uniform":
        return rng.uniform(0.05, HALF_PI - 0.05, size=cfg.B)
    if cfg.t_mode == "edges":
        t = np.empty(cfg.B)
        lo = cfg.B // 2
        t[:lo] = rng.uniform(0.01, 0.1, size=lo)
        t[lo:] = rng.uniform(HALF_PI - 0.1, HALF_PI - 0.01, size=cfg.B - lo)
        return t
    raise ValueError(cfg.t_mode)


def make_mask(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    m = np.zeros((cfg.B, cfg.Nt), dtype=np.uint8)
    if cfg.mask_mode == "prefix":
        m[:, : cfg.Ntv] = 1
    elif cfg.mask_mode == "scatter":
        # per-sample random valid sets; sample b keeps max(1, Ntv - b) tokens
        for b in range(cfg.B):
            n = max(0, min(cfg.Nt, cfg.Ntv - b))
            idx = rng.choice(cfg.Nt, size=n, replace=False)
            m[b, idx] = 1
    else:
        raise ValueError(cfg.mask_mode)
    return m


def make_data(cfg: Config) -> dict:
    """Latents, noise, text, mask and timesteps (seed 100+index).

    Draw order: z0_v, z0_a, eps_v, eps_a, text, t (then the scatter mask, if any).
    Padded text positions hold N(0,1) values like valid ones, so a kernel that
    ignores the mask produces different results.
    """
    rng = np.random.default_rng(100 + cfg.index)
    z0_v = rng.standard_normal((cfg.B, cfg.Nv, cfg.Cv)) * cfg.z0_scale_v
    z0_a = rng.standard_normal((cfg.B, cfg.Na, cfg.Ca)) * cfg.z0_scale_a
    eps_v = rng.standard_normal((cfg.B, cfg.Nv, cfg.Cv))
    eps_a = rng.standard_normal((cfg.B, cfg.Na, cfg.Ca))
    text = rng.standard_normal((cfg.B, cfg.Nt, cfg.d))
    t = draw_t(cfg, rng)
    mask = make_mask(cfg, rng)
    dt = cfg.in_dtype
    return dict(z0_v=round_to(z0_v, dt), z0_a=round_to(z0_a, dt),
                eps_v=round_to(eps_v, dt), eps_a=round_to(eps_a, dt),
                text=round_to(text, dt), text_mask=mask, t=t)


def make_weights(cfg: Config, which: str) -> dict:
    """One seeded copy of the joint block (teacher: seed 200+index, student:
    300+index, the DMD fake-score block: 400+index).

    Draw order: w_in_v, w_in_a, w_t, w_qkv, w_out_v, w_out_a; each ~ N(0, 1/fan_in).
    """
    seed = {"teacher": 200, "student": 300, "fake": 400}[which] + cfg.index
    rng = np.random.default_rng(seed)
    d = cfg.d

    def lin(out_f, in_f):
        return rng.standard_normal((out_f, in_f)) / math.sqrt(in_f)

    w = dict(w_in_v=lin(d, cfg.Cv), w_in_a=lin(d, cfg.Ca), w_t=lin(d, d), w_qkv=lin(3 * d, d),
             w_out_v=lin(cfg.Cv, d), w_out_a=lin(cfg.Ca, d))
    return {k: round_to(v, cfg.in_dtype) for k, v in w.items()}


def make_problem(cfg: Config) -> dict:
    """Everything one call of the sCM target consumes."""
    return dict(cfg=cfg, data=make_data(cfg), teacher=make_weights(cfg, "teacher"),
                student=make_weights(cfg, "student"))


def make_dmd_data(cfg: Config) -> dict:
    """Inputs of the joint DMD term (seed 500+index).

    The student's generated paired sample x0_hat (drawn like the data latents,
    with the same per-modality scales), fresh noise, and timesteps drawn like
    the sCM ones.  Draw order: x0_v, x0_a, eps_v, eps_a, t.  The text and its
    mask are the sCM batch's own (``make_data``): both terms share the batch's
    condition.
    """
    rng = np.random.default_rng(500 + cfg.index)
    x0_v = rng.standard_normal((cfg.B, cfg.Nv, cfg.Cv)) * cfg.z0_scale_v
    x0_a = rng.standard_normal((cfg.B, cfg.Na, cfg.Ca)) * cfg.z0_scale_a
    eps_v = rng.standard_normal((cfg.B, cfg.Nv, cfg.Cv))
    eps_a = rng.standard_normal((cfg.B, cfg.Na, cfg.Ca))
    t = draw_t(cfg, rng)
    dt = cfg.in_dtype
    return dict(x0_v=round_to(x0_v, dt), x0_a=round_to(x0_a, dt), eps_v=round_to(eps_v, dt),
                eps_a=round_to(eps_a, dt), t=t)


def make_dmd_problem(cfg: Config, data: dict | None = None) -> dict:
    """Everything one call of the DMD term consumes: its own sample, noise and
    timesteps, the sCM batch's text and mask, the teacher and the fake-score block."""
    data = make_data(cfg) if data is None else data
    dmd = make_dmd_data(cfg)
    dmd["text"] = data["text"]
    dmd["text_mask"] = data["text_mask"]
    return dict(cfg=cfg, data=dmd, teacher=make_weights(cfg, "teacher"),
                fake=make_weights(cfg, "fake"))


def make_attention_operands(B: int, H: int, dh: int, Nq: int, Nk: int, seed: int,
                            nk_valid=None, q_scale: float = 1.0, dtype=np.float64,
                            k_scale: float = 1.0, tangent_scale: float = 1.0) -> dict:
    """Random bf16-valued attention operands in sequence-major layout [B, N, H, dh].

    Queries are the first Nq rows of the same token sequence the keys span
    (Nq <= Nk).  ``nk_valid[b]`` keys are valid for sample b; key rows past it
    hold random values so that an unmasked kernel is caught.
    """
    rng = np.random.default_rng(seed)
    sh_q = (B, Nq, H, dh)
    sh_k = (B, Nk, H, dh)

    def draw(shape, s=1.0):
        x = rng.standard_normal(shape, dtype=np.float32 if dtype == np.float32 else np.float64)
        return round_bf16(x * s).astype(dtype)

    q = draw(sh_q, q_scale)
    k = draw(sh_k, k_scale)
    v = draw(sh_k)
    qd = draw(sh_q, tangent_scale)
    kd = draw(sh_k, tangent_scale)
    vd = draw(sh_k, tangent_scale)
    if nk_valid is None:
        nk_valid = np.full(B, Nk, dtype=np.int32)
    return dict(q=q, k=k, v=v, qd=qd, kd=kd, vd=vd, nk=np.asarray(nk_valid, dtype=np.int32))
