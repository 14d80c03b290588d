"""Seeded synthetic workloads for quantized attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no softmax, no attention, none of the method's
quantizers).  The one encoding it does is input synthesis: the FP8 decode
cache is built from float draws with torch's float8_e4m3fn cast and a
per-token amax / 448 scale, because a paged cache arrives already encoded
(the MXFP4 cache is drawn directly as E2M1 codes and E8M0 exponents).  Both the CPU oracle and the HIP path read the
arrays it returns, so the two sides always see the same inputs.

Every tensor is drawn with ``numpy.random.default_rng([config_id, tensor_id])``
(tensor ids: Q=0, K=1, V=2, K channel offset=3, outlier channels=4, pages=5),
sampled in float32 and cast round-to-nearest-even to the workload's dtype by
torch.

Workloads (the shapes the pages discuss; the pages give no data sets):

* ``tiny``        B=1, H=2, L=256, D=64, fp16, Q/K/V ~ N(0,1), K += per-channel
                  offset ~ N(0, 2^2), non-causal.
* ``llm_prefill`` B=2, H=32, L=4096, D=128, bf16, K offset ~ N(0, 3^2), causal.
* ``video_dit``   B=1, H=40, L=32760, D=128, bf16, Q/K Student-t(3) with 4
                  outlier channels per head scaled x20 (same channels for Q and
                  K), V ~ N(0,1); Q/K/V are strided [B,L,H,D] views into one
                  stacked [B,L,3,H,D] buffer (the layout a fused QKV projection
                  produces, which FastVideo's sage_attn3 backend copies with a
                  permute+contiguous before its kernel).
* ``video_dit_mxfp4`` same tensors as ``video_dit`` (MXFP4 QK with Hadamard).
* ``paged_decode`` batch 16, 4 query tokens per sequence, 16 query heads on 1
                  KV head, D=128, bf16 queries; FP8 e4m3 KV cache with a
                  per-token fp32 scale, page 128, context 8192, sliding window
                  4096, page table = seeded permutation of the 1024-page pool.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

T_Q, T_K, T_V, T_OFFSET, T_OUTLIER, T_PAGES = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    config_id: int          # seed root
    B: int
    H: int
    Lq: int
    Lk: int
    D: int
    dtype: torch.dtype
    causal: bool
    qk_mode: str            # "int8" or "mxfp4"
    dist: str               # "normal_offset" or "student_t_outliers"
    k_offset_sigma: float = 0.0
    stacked: bool = False   # Q/K/V are views of a stacked [B,L,3,H,D] buffer
    outlier_channels: int = 4
    outlier_scale: float = 20.0
    q_block: int = 128
    k_block: int = 64

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    config_id: int
    batch: int
    mtp: int
    hq: int
    hkv: int
    D: int
    page_size: int
    ctx: int
    window: int
    q_dtype: torch.dtype = torch.bfloat16

    @property
    def pages_per_seq(self) -> int:
        return (self.ctx + self.page_size - 1) // self.page_size

    @property
    def num_pages(self) -> int:
        return self.batch * self.pages_per_seq

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


WORKLOADS = {
    "tiny": PrefillWorkload("tiny", 0, 1, 2, 256, 256, 64, torch.float16, False, "int8",
                            "normal_offset", k_offset_sigma=2.0),
    "llm_prefill": PrefillWorkload("llm_prefill", 1, 2, 32, 4096, 4096, 128, torch.bfloat16,
                                   True, "int8", "normal_offset", k_offset_sigma=3.0),
    "video_dit": PrefillWorkload("video_dit", 2, 1, 40, 32760, 32760, 128, torch.bfloat16,
                                 False, "int8", "student_t_outliers", stacked=True),
    "video_dit_mxfp4": PrefillWorkload("video_dit_mxfp4", 2, 1, 40, 32760, 32760, 128,
                                       torch.bfloat16, False, "mxfp4", "student_t_outliers",
                                       stacked=True),
    "paged_decode": DecodeWorkload("paged_decode", 4, 16, 4, 16, 1, 128, 128, 8192, 4096),
}


def _rng(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([config_id, tensor_id])


def _normal(config_id, tensor_id, shape) -> np.ndarray:
    return _rng(config_id, tensor_id).standard_normal(shape, dtype=np.float32)


def _student_t(config_id, tensor_id, shape, nu=3.0, chunk=1 << 24) -> np.ndarray:
    rng = _rng(config_id, tensor_id)
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = rng.standard_t(nu, e - s).astype(np.float32)
    return out.reshape(shape)


def outlier_channels(w: PrefillWorkload) -> np.ndarray:
    """[H, n] distinct channel indices per head (same for Q and K)."""
    rng = _rng(w.config_id, T_OUTLIER)
    return np.stack([rng.choice(w.D, size=w.outlier_channels, replace=False)
                     for _ in range(w.H)]).astype(np.int64)


def _to_dtype(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(a).to(dtype)


@dataclass
class PrefillInputs:
    q: torch.Tensor                  # logical [B, Lq, H, D] (possibly strided view)
    k: torch.Tensor                  # logical [B, Lk, H, D]
    v: torch.Tensor                  # logical [B, Lk, H, D]
    base: Optional[torch.Tensor] = None  # stacked buffer when the views share one


def make_prefill(w: PrefillWorkload, Lq: Optional[int] = None, Lk: Optional[int] = None,
                 device: str = "cpu", B: Optional[int] = None,
                 H: Optional[int] = None) -> PrefillInputs:
    """Draws Q, K, V for a prefill workload.

    ``Lq``/``Lk``/``B``/``H`` override the sizes (same distributions and seeds;
    a smaller draw is its own sample, not a slice of the full one), which the
    parity tests use for sizes the oracle finishes quickly.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    D = w.D
    Lq = w.Lq if Lq is None else Lq
    Lk = w.Lk if Lk is None else Lk
    cid = w.config_id
    if w.dist == "normal_offset":
        q = _normal(cid, T_Q, (B, Lq, H, D))
        k = _normal(cid, T_K, (B, Lk, H, D))
        v = _normal(cid, T_V, (B, Lk, H, D))
        off = _rng(cid, T_OFFSET).normal(0.0, w.k_offset_sigma, (H, D)).astype(np.float32)
        k += off[None, None, :, :]
    elif w.dist == "student_t_outliers":
        q = _student_t(cid, T_Q, (B, Lq, H, D))
        k = _student_t(cid, T_K, (B, Lk, H, D))
        v = _normal(cid, T_V, (B, Lk, H, D))
        ch = outlier_channels(w)
        for h in range(min(H, ch.shape[0])):
            q[:, :, h, ch[h]] *= np.float32(w.outlier_scale)
            k[:, :, h, ch[h]] *= np.float32(w.outlier_scale)
    else:
        raise ValueError(w.dist)

    if w.stacked and Lq == Lk:
        base = torch.empty((B, Lq, 3, H, D), dtype=w.dtype)
        base[:, :, 0] = _to_dtype(q, w.dtype)
        del q
        base[:, :, 1] = _to_dtype(k, w.dtype)
        del k
        base[:, :, 2] = _to_dtype(v, w.dtype)
        del v
        if device != "cpu":
            base = base.to(device)
        return PrefillInputs(base[:, :, 0], base[:, :, 1], base[:, :, 2], base)
    qt, kt, vt = (_to_dtype(x, w.dtype) for x in (q, k, v))
    if device != "cpu":
        qt, kt, vt = qt.to(device), kt.to(device), vt.to(device)
    return PrefillInputs(qt, kt, vt)


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [batch, mtp, hq, D] bf16
    k_cache: torch.Tensor      # [num_pages, hkv, page, D] uint8 (e4m3 codes)
    v_cache: torch.Tensor      # [num_pages, hkv, page, D] uint8 (e4m3 codes)
    k_scale: torch.Tensor      # [num_pages, hkv, page] fp32
    v_scale: torch.Tensor      # [num_pages, hkv, page] fp32
    page_table: torch.Tensor   # [batch, pages_per_seq] int32
    ctx_lens: torch.Tensor     # [batch] int32


def _per_token_e4m3(x: np.ndarray):
    """Synthesises an e4m3 cache with a per-token fp32 scale (amax/448) from
    float draws, using torch's float8_e4m3fn cast.  This builds an input; the
    decode path consumes the cache as given."""
    t = torch.from_numpy(x)
    amax = t.abs().amax(dim=-1, keepdim=True)
    scale = (amax / 448.0).to(torch.float32)
    scale = torch.where(scale > 0, scale, torch.ones_like(scale))
    codes = (t / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.squeeze(-1).contiguous()


@dataclass
class DecodeInputsMX:
    """MXFP4 KV cache, one E2M1 code (0-15, sign in bit 3) per byte; V
    transposed.  `packed()` gives the two-codes-per-byte tensors the library
    takes (element 2i in the low nibble)."""
    q: torch.Tensor            # [batch, mtp, hq, D] bf16
    k_codes: torch.Tensor      # [num_pages, hkv, page, D] uint8
    k_e8: torch.Tensor         # [num_pages, hkv, page, D / 32] uint8 (E8M0)
    v_codes: torch.Tensor      # [num_pages, hkv, D, page] uint8
    v_e8: torch.Tensor         # [num_pages, hkv, D, page / 32] uint8 (E8M0)
    page_table: torch.Tensor   # [batch, pages_per_seq] int32
    ctx_lens: torch.Tensor     # [batch] int32

    def packed(self):
        pk = lambda c: (c[..., 0::2] | (c[..., 1::2] << 4)).contiguous()
        return pk(self.k_codes), pk(self.v_codes)


# magnitude index 0..7 of E2M1 (0, 0.5, 1, 1.5, 2, 3, 4, 6) drawn with these
# weights, a uniform sign, and block exponents around 2^-1: roughly the codes
# of N(0, 1) values in blocks of 32 (synthetic codes, no quantization here)
_E2M1_WEIGHTS = np.array([0.10, 0.20, 0.20, 0.16, 0.14, 0.12, 0.06, 0.02])


def _mx_codes(rng: np.random.Generator, shape) -> np.ndarray:
    mag = rng.choice(8, size=shape, p=_E2M1_WEIGHTS / _E2M1_WEIGHTS.sum())
    sign = rng.integers(0, 2, size=shape)
    return (mag | (sign << 3)).astype(np.uint8)


def _mx_exponents(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.choice(np.array([125, 126, 127], np.uint8), size=shape, p=[0.1, 0.8, 0.1])


def make_decode_mx(w: DecodeWorkload, batch: Optional[int] = None, ctx: Optional[int] = None,
                   pool_seed: int = 0) -> DecodeInputsMX:
    """Draws a paged decode problem over an MXFP4 cache of the same shape as
    make_decode's (same queries, page table and lengths)."""
    batch = w.batch if batch is None else batch
    ctx = w.ctx if ctx is None else ctx
    pps = (ctx + w.page_size - 1) // w.page_size
    npages = batch * pps
    cid = w.config_id if pool_seed == 0 else 1000 + pool_seed
    q = _normal(w.config_id, T_Q, (batch, w.mtp, w.hq, w.D))
    rk, rv = _rng(cid, T_K), _rng(cid, T_V)
    kc = _mx_codes(rk, (npages, w.hkv, w.page_size, w.D))
    ke = _mx_exponents(rk, (npages, w.hkv, w.page_size, w.D // 32))
    vc = _mx_codes(rv, (npages, w.hkv, w.D, w.page_size))
    ve = _mx_exponents(rv, (npages, w.hkv, w.D, w.page_size // 32))
    perm = _rng(cid, T_PAGES).permutation(npages).astype(np.int32)
    table = torch.from_numpy(perm.reshape(batch, pps).copy())
    ctx_lens = torch.full((batch,), ctx, dtype=torch.int32)
    t = torch.from_numpy
    return DecodeInputsMX(_to_dtype(q, w.q_dtype), t(kc), t(ke), t(vc), t(ve), table, ctx_lens)


def make_decode(w: DecodeWorkload, batch: Optional[int] = None, ctx: Optional[int] = None,
                pool_seed: int = 0) -> DecodeInputs:
    """Draws a paged decode problem.  ``pool_seed`` > 0 draws an independent KV
    pool and page table of the same shape (used to rotate pools when timing)."""
    batch = w.batch if batch is None else batch
    ctx = w.ctx if ctx is None else ctx
    pps = (ctx + w.page_size - 1) // w.page_size
    npages = batch * pps
    cid = w.config_id if pool_seed == 0 else 1000 + pool_seed
    q = _normal(w.config_id, T_Q, (batch, w.mtp, w.hq, w.D))
    kf = _normal(cid, T_K, (npages, w.hkv, w.page_size, w.D))
    vf = _normal(cid, T_V, (npages, w.hkv, w.page_size, w.D))
    kc, ks = _per_token_e4m3(kf)
    vc, vs = _per_token_e4m3(vf)
    perm = _rng(cid, T_PAGES).permutation(npages).astype(np.int32)
    table = torch.from_numpy(perm.reshape(batch, pps).copy())
    ctx_lens = torch.full((batch,), ctx, dtype=torch.int32)
    return DecodeInputs(_to_dtype(q, w.q_dtype), kc, vc, ks, vs, table, ctx_lens)
