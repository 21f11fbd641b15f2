"""Seeded synthetic workloads: pool initial states and per-step decode inputs.

This module only draws random numbers and shapes them; it holds none of the
state-update arithmetic.  Both the HIP path (through the tests and the
benchmark) and the fp64 CPU oracle consume exactly the arrays it returns.

The workloads stand in for the model states the SinkState paper measures
(Nemotron-3-Nano-4B: 21 Mamba-2 layers x 96 heads of 80x128 states at batch
128, i.e. 258,048 states; Qwen GDN layers with 128x128 states), which need
model weights and datasets that are not used here.  The "linear attention
sink" (SinkState 3.1: queries, keys and values concentrate in a stable
low-dimensional subspace) is modelled by drawing q, k, v mostly from a fixed
per-head subspace plus isotropic noise.

Orientation: a state is S (d_k x d_v), o = S^T q.  The paper's "80x128"
Mamba-2 state is H = S^T with d_v = 80 (head dim) and d_k = 128 (state dim).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

BASE_SEED = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int
    n_requests: int
    n_layers: int
    n_heads: int
    d_k: int
    d_v: int
    steps: int
    K: int = 8
    r: int = 8
    kind: str = "scalar"          # scalar | delta | mixed
    eps_scalar: float = 3e-3
    eps_delta: float = 1e-2
    init: str = "aligned8"        # empty | aligned8 | random_rank | mixed_rank
    inputs: str = "split70"       # shared4 | split70 | sub6
    alpha_lo: float = 0.95
    stagger: str = "even4"        # none | even4 | paper8 | state8
    decay: str = "scalar"         # scalar: one alpha per state | channel: one per key channel ([N][d_k])
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_states(self) -> int:
        return self.n_requests * self.n_layers * self.n_heads

    @property
    def heads_per_request(self) -> int:
        return self.n_layers * self.n_heads

    @property
    def diag_decay(self) -> bool:
        return self.decay == "channel"

    def scaled(self, n_requests: int) -> "Workload":
        return replace(self, n_requests=int(n_requests))


# The workloads.  Where the pages leave a detail open, the comment on each states the reading taken.
WORKLOADS = {
    # 64 fp32 states, d_k=16, d_v=32, one shared 4-dim subspace, sigma_noise 0.05,
    # unit keys, empty start, eps 1e-3, compaction whenever the pad fills.
    "tiny": Workload("tiny", 1, n_requests=1, n_layers=1, n_heads=64, d_k=16, d_v=32, steps=256,
                     kind="scalar", eps_scalar=1e-3, init="empty", inputs="shared4", alpha_lo=0.90,
                     stagger="none", description="64 scalar-decay states 16x32, 256 steps"),
    # 128 requests x 21 layers x 96 heads = 258,048 Mamba-2 states, d_k=128, d_v=80.
    "mamba2_258k": Workload("mamba2_258k", 2, n_requests=128, n_layers=21, n_heads=96, d_k=128, d_v=80,
                            steps=1024, kind="scalar", eps_scalar=3e-3, init="aligned8", inputs="split70",
                            alpha_lo=0.95, stagger="even4",
                            description="258,048 Mamba-2 states 128x80 (d_k x d_v), rank-8 start"),
    # 64 requests x 24 layers x 64 heads = 98,304 Gated-DeltaNet states 128x128.
    "gdn_delta": Workload("gdn_delta", 3, n_requests=64, n_layers=24, n_heads=64, d_k=128, d_v=128, steps=512,
                          kind="delta", eps_delta=1e-2, init="random_rank", inputs="sub6", alpha_lo=0.90,
                          stagger="paper8", description="98,304 delta-rule states 128x128"),
    # 32,768 mixed states 128x80: half scalar, half delta, ranks 2..64 log-uniform
    # plus 0..24 small frozen extras; above 49 components a state is dense.
    "mixed_dense": Workload("mixed_dense", 4, n_requests=32, n_layers=16, n_heads=64, d_k=128, d_v=80, steps=256,
                            kind="mixed", eps_scalar=3e-3, eps_delta=1e-2, init="mixed_rank", inputs="mixed",
                            alpha_lo=0.95, stagger="state8",
                            description="32,768 mixed-rule states 128x80 with a dense fallback"),
    # 512 requests x 2016 = 1,032,192 Mamba-2 states, as mamba2_258k.
    "mamba2_1m": Workload("mamba2_1m", 5, n_requests=512, n_layers=21, n_heads=96, d_k=128, d_v=80, steps=128,
                          kind="scalar", eps_scalar=3e-3, init="aligned8", inputs="split70", alpha_lo=0.95,
                          stagger="even4", description="1,032,192 Mamba-2 states 128x80"),
    # Kimi Delta Attention (per-channel decay): 64 requests x 20 layers x 32 heads = 40,960 states
    # 128x128 (Kimi-Linear's KDA layers, SEED section 5), delta rule, inputs and initial ranks as
    # gdn_delta, each key channel's decay drawn from U(0.9, 1.0) every step.
    "kda_delta": Workload("kda_delta", 6, n_requests=64, n_layers=20, n_heads=32, d_k=128, d_v=128, steps=512,
                          kind="delta", eps_delta=1e-2, init="random_rank", inputs="sub6", alpha_lo=0.90,
                          stagger="paper8", decay="channel",
                          description="40,960 Kimi Delta Attention states 128x128, per-channel decay"),
}


def get(name: str, n_requests: int | None = None) -> Workload:
    w = WORKLOADS[name]
    return w if n_requests is None else w.scaled(n_requests)


# --------------------------------------------------------------------------
# structure: layer / head / group of each state
# --------------------------------------------------------------------------
def state_layout(w: Workload):
    """state s = (b * n_layers + l) * n_heads + h  ->  (layer, head index within the request)."""
    s = np.arange(w.n_states, dtype=np.int64)
    within = s % w.heads_per_request          # l * n_heads + h
    layer = within // w.n_heads
    return layer, within


def groups(w: Workload):
    """Compaction groups and their step offsets (staggered compaction)."""
    layer, _ = state_layout(w)
    s = np.arange(w.n_states, dtype=np.int64)
    if w.stagger == "none":
        g = np.zeros(w.n_states, np.int32)
        offs = np.array([0], np.int32)
    elif w.stagger == "even4":      # 4 groups of layers, offsets 0,2,4,6: 1/4 of layers on every even step
        g = (layer % 4).astype(np.int32)
        offs = np.array([0, 2, 4, 6], np.int32)
    elif w.stagger == "paper8":     # layer l gets offset l mod K
        g = (layer % w.K).astype(np.int32)
        offs = np.arange(w.K, dtype=np.int32)
    elif w.stagger == "state8":     # state s gets offset s mod K
        g = (s % w.K).astype(np.int32)
        offs = np.arange(w.K, dtype=np.int32)
    else:
        raise ValueError(w.stagger)
    return g, offs


def rules(w: Workload):
    if w.kind == "scalar":
        return np.zeros(w.n_states, np.uint8)
    if w.kind == "delta":
        return np.ones(w.n_states, np.uint8)
    return (np.arange(w.n_states) % 2).astype(np.uint8)   # mixed: odd states use the delta rule


def eps_of(w: Workload):
    rl = rules(w)
    return np.where(rl == 1, w.eps_delta, w.eps_scalar).astype(np.float32)


# --------------------------------------------------------------------------
# random helpers (float64 on the host, then rounded once to float32)
# --------------------------------------------------------------------------
def _gen(seed: int, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    return g


def _orthonormal(gen, batch, d, m):
    """batch x d x m with orthonormal columns (QR of a Gaussian, sign-fixed)."""
    a = torch.randn(batch, d, m, generator=gen, dtype=torch.float64)
    q, r = torch.linalg.qr(a)
    sgn = torch.sign(torch.diagonal(r, dim1=-2, dim2=-1))
    sgn[sgn == 0] = 1.0
    return q * sgn.unsqueeze(-2)


def head_bases(w: Workload, seed: int = BASE_SEED):
    """Per-head key-side and value-side subspace bases, float64 on the host."""
    gen = _gen(seed * 7919 + w.seed_id)
    if w.inputs == "shared4":
        Pk = _orthonormal(gen, 1, w.d_k, 4).expand(w.heads_per_request, -1, -1).contiguous()
        Pv = _orthonormal(gen, 1, w.d_v, 4).expand(w.heads_per_request, -1, -1).contiguous()
        return {"Pk": Pk, "Pv": Pv}
    m8 = 8
    out = {"Pk": _orthonormal(gen, w.heads_per_request, w.d_k, m8),
           "Pv": _orthonormal(gen, w.heads_per_request, w.d_v, m8)}
    if w.inputs in ("sub6", "mixed"):
        out["Pk6"] = _orthonormal(gen, w.heads_per_request, w.d_k, 6)
        out["Pv6"] = _orthonormal(gen, w.heads_per_request, w.d_v, 6)
    return out


# --------------------------------------------------------------------------
# initial states
# --------------------------------------------------------------------------
def initial_state(w: Workload, seed: int = BASE_SEED):
    """Initial factors in CSR form (float32) plus rules, eps and groups.

    Returns a dict with comp_off (int64 [N+1]), u ([T, d_k]), v ([T, d_v]),
    sigma ([T]), rule (uint8 [N]), eps (float32 [N]), group_of_state (int32
    [N]), group_offset (int32 [G]).  Components of a state are sorted by sigma.
    """
    N, dk, dv = w.n_states, w.d_k, w.d_v
    gen = _gen(seed * 104729 + w.seed_id)
    grp, offs = groups(w)
    base = {"rule": rules(w), "eps": eps_of(w), "group_of_state": grp, "group_offset": offs}
    if w.init == "empty":
        base.update(comp_off=np.zeros(N + 1, np.int64), u=np.zeros((0, dk), np.float32),
                    v=np.zeros((0, dv), np.float32), sigma=np.zeros(0, np.float32))
        return base
    _, head = state_layout(w)
    if w.init == "aligned8":
        # rank 8 aligned with the head's subspace, sigma_i = 0.5^i; built in chunks
        B = head_bases(w, seed)
        u = np.empty((N * 8, dk), np.float32)
        v = np.empty((N * 8, dv), np.float32)
        hidx_all = torch.from_numpy(head)
        chunk = 1 << 16
        for a in range(0, N, chunk):
            b = min(N, a + chunk)
            R1 = _orthonormal(gen, b - a, 8, 8)
            R2 = _orthonormal(gen, b - a, 8, 8)
            hidx = hidx_all[a:b]
            U = torch.matmul(B["Pk"][hidx], R1)          # n x dk x 8
            V = torch.matmul(B["Pv"][hidx], R2)          # n x dv x 8
            u[a * 8:b * 8] = U.transpose(1, 2).reshape(-1, dk).to(torch.float32).numpy()
            v[a * 8:b * 8] = V.transpose(1, 2).reshape(-1, dv).to(torch.float32).numpy()
        sig = (0.5 ** np.arange(8, dtype=np.float64)).astype(np.float32)
        base.update(comp_off=np.arange(N + 1, dtype=np.int64) * 8, u=u, v=v, sigma=np.tile(sig, N))
        return base
    if w.init == "random_rank":
        # rank ~ U{2..16}, random orthonormal factors, sigma log-spaced from 1 to 2*eps
        ranks = torch.randint(2, 17, (N,), generator=gen).numpy()
        U = _orthonormal(gen, N, dk, 16)
        V = _orthonormal(gen, N, dv, 16)
        return _pack(base, ranks, U, V, [np.logspace(0.0, math.log10(2 * float(base["eps"][i])), int(ranks[i]))
                                         for i in range(N)], dk, dv)
    if w.init == "mixed_rank":
        # target rank log-uniform in [2, 64] with sigma log-spaced 1 -> 0.05, plus 0..24
        # extra non-orthogonal unit components with sigma log-uniform in [1.5 eps, 0.05)
        lr = torch.rand(N, generator=gen, dtype=torch.float64) * (math.log(64) - math.log(2)) + math.log(2)
        ranks = torch.round(torch.exp(lr)).to(torch.int64).clamp(2, 64).numpy()
        extras = torch.randint(0, 25, (N,), generator=gen).numpy()
        U = _orthonormal(gen, N, dk, 64)
        V = _orthonormal(gen, N, dv, 64)
        eu = torch.randn(N, dk, 24, generator=gen, dtype=torch.float64)
        ev = torch.randn(N, dv, 24, generator=gen, dtype=torch.float64)
        eu = eu / eu.norm(dim=1, keepdim=True)
        ev = ev / ev.norm(dim=1, keepdim=True)
        ux = torch.rand(N, 24, generator=gen, dtype=torch.float64).numpy()
        sig_list, Ufull, Vfull = [], [], []
        tot = ranks + extras
        U = torch.cat([U, eu], dim=2)
        V = torch.cat([V, ev], dim=2)
        for i in range(N):
            e = float(base["eps"][i])
            main = np.logspace(0.0, math.log10(0.05), int(ranks[i]))
            lo, hi = math.log(1.5 * e), math.log(0.05)
            ext = np.sort(np.exp(lo + (hi - lo) * ux[i, :int(extras[i])]))[::-1]
            sig_list.append(np.concatenate([main, ext]))
        cols = [np.concatenate([np.arange(int(ranks[i])), 64 + np.arange(int(extras[i]))]) for i in range(N)]
        return _pack(base, tot, U, V, sig_list, dk, dv, cols=cols)
    raise ValueError(w.init)


def _pack(base, ranks, U, V, sig_list, dk, dv, cols=None):
    N = len(ranks)
    off = np.zeros(N + 1, np.int64)
    off[1:] = np.cumsum(ranks)
    T = int(off[-1])
    u = np.zeros((T, dk), np.float32)
    v = np.zeros((T, dv), np.float32)
    s = np.zeros(T, np.float32)
    Un = U.numpy()
    Vn = V.numpy()
    for i in range(N):
        c = np.arange(int(ranks[i])) if cols is None else cols[i]
        a, b = off[i], off[i + 1]
        u[a:b] = Un[i][:, c].T
        v[a:b] = Vn[i][:, c].T
        s[a:b] = sig_list[i]
    base.update(comp_off=off, u=u, v=v, sigma=s)
    return base


# --------------------------------------------------------------------------
# per-step inputs
# --------------------------------------------------------------------------
class StepInputs:
    """Per-step q, k, v, alpha, beta for every state (or a subset), float32.

    Draws come from torch generators seeded by (seed, config, step), so a step's
    inputs are reproducible on a given device type.  The per-head bases are
    drawn once on the host in float64 and used in float32 on the device.
    """

    def __init__(self, w: Workload, seed: int = BASE_SEED, device="cpu"):
        self.w = w
        self.seed = int(seed)
        self.device = torch.device(device)
        B = head_bases(w, seed)
        self.B = {k: v.to(torch.float32).to(self.device) for k, v in B.items()}
        _, head = state_layout(w)
        self.head = torch.from_numpy(head).to(self.device)
        self.rule = torch.from_numpy(rules(w).astype(np.int64)).to(self.device)

    def _proj(self, P, g, idx):
        # x[s] = P[head(s)] @ g[s]
        if idx is None and P.shape[0] == self.w.heads_per_request:
            H = P.shape[0]
            nb = g.shape[0] // H
            gh = g.view(nb, H, -1).permute(1, 2, 0).contiguous()       # H x m x nb
            x = torch.bmm(P, gh)                                       # H x d x nb
            return x.permute(2, 0, 1).reshape(g.shape[0], -1).contiguous()
        hh = self.head if idx is None else self.head[idx]
        return torch.matmul(P[hh], g.unsqueeze(-1)).squeeze(-1)

    def generate(self, step: int, states=None):
        w = self.w
        idx = None if states is None else torch.as_tensor(states, dtype=torch.int64, device=self.device)
        n = w.n_states if idx is None else int(idx.shape[0])
        gen = _gen(self.seed * 1_000_003 + w.seed_id * 65_537 + int(step), self.device)
        dev, f32 = self.device, torch.float32
        dk, dv = w.d_k, w.d_v
        ashape = (n, dk) if w.diag_decay else (n,)  # per-channel decay: one alpha per key channel
        alpha = w.alpha_lo + (1.0 - w.alpha_lo) * torch.rand(ashape, generator=gen, device=dev, dtype=f32)
        beta = torch.sigmoid(torch.randn(n, generator=gen, device=dev, dtype=f32))

        def draw(m, d):
            return (torch.randn(n, m, generator=gen, device=dev, dtype=f32),
                    torch.randn(n, d, generator=gen, device=dev, dtype=f32))

        if w.inputs == "shared4":
            (gk, nk), (gq, nq), (gv, nv) = draw(4, dk), draw(4, dk), draw(4, dv)
            k = self._proj(self.B["Pk"], gk, idx) + 0.05 * nk
            q = self._proj(self.B["Pk"], gq, idx) + 0.05 * nq
            v = self._proj(self.B["Pv"], gv, idx) + 0.05 * nv
            k = k / k.norm(dim=1, keepdim=True)
        elif w.inputs == "split70":
            k, q, v = self._split70(draw, idx, dk, dv)
        elif w.inputs == "sub6":
            k, q, v = self._sub6(draw, idx, dk, dv)
        elif w.inputs == "mixed":
            k1, q1, v1 = self._split70(draw, idx, dk, dv)
            k2, q2, v2 = self._sub6(draw, idx, dk, dv)
            rl = (self.rule if idx is None else self.rule[idx]).unsqueeze(1).to(torch.bool)
            k = torch.where(rl, k2, k1)
            q = torch.where(rl, q2, q1)
            v = torch.where(rl, v2, v1)
        else:
            raise ValueError(w.inputs)
        return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(), "alpha": alpha.contiguous(),
                "beta": beta.contiguous()}

    def _split70(self, draw, idx, dk, dv):
        # energy split: 70% from the head's 8-dim subspace, 30% isotropic (E|x|^2 = 1)
        a, b = math.sqrt(0.7 / 8.0), math.sqrt(0.3)
        (gk, nk), (gq, nq), (gv, nv) = draw(8, dk), draw(8, dk), draw(8, dv)
        k = a * self._proj(self.B["Pk"], gk, idx) + (b / math.sqrt(dk)) * nk
        q = a * self._proj(self.B["Pk"], gq, idx) + (b / math.sqrt(dk)) * nq
        v = a * self._proj(self.B["Pv"], gv, idx) + (b / math.sqrt(dv)) * nv
        return k, q, v

    def _sub6(self, draw, idx, dk, dv):
        # per-head 6-dim subspace plus noise sigma = 0.1, unit keys
        (gk, nk), (gq, nq), (gv, nv) = draw(6, dk), draw(6, dk), draw(6, dv)
        k = self._proj(self.B["Pk6"], gk, idx) + 0.1 * nk
        q = self._proj(self.B["Pk6"], gq, idx) + 0.1 * nq
        v = self._proj(self.B["Pv6"], gv, idx) + 0.1 * nv
        k = k / k.norm(dim=1, keepdim=True)
        return k, q, v
