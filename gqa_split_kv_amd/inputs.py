"""Seeded synthetic inputs for GQA decode (shared by the tests, the smoke check and
the benchmark).

This module only draws and lays out input data; it holds none of the method's
arithmetic and imports neither the HIP binding nor the oracle.

Layouts (row-major, contiguous):
  q, o      [batch, h_q, d], or [batch, t_q, h_q, d] with t_q query tokens per sequence
  k, v      [sum(seq_lens), h_kv, d]   sequences packed back to back
  seq_lens  int32[batch]

Element values are i.i.d. N(0, 1) drawn in float32 and rounded to bf16 or
IEEE fp16 (round-to-nearest-even) for the 16-bit workloads; the fp32 workload
keeps the float32 draws.  The long-context stress workload scales a random 0.1% of the
key rows of every sequence (all kv heads of that row) by 8, which makes the
softmax peaked.

Two generators:
  * host_case   -- numpy PCG64, bit-reproducible on any machine; used for every
                   workload the CPU oracle covers whole (small shapes, configs 1-3).
  * device_case -- torch's device generator (Philox) seeded per tensor; used for
                   the multi-GiB workloads (configs 4-5).  Reproducible for a given
                   torch build and device type.  Host copies of the rows the oracle
                   needs are taken from the device tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------------------
# The five workloads.  All decode one query token per sequence, scale = 1/sqrt(d).
# --------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    dtype: str               # "bf16", "f16" or "f32" (inputs; the accumulator is always fp32)
    batch: int
    h_q: int
    h_kv: int
    d: int
    seq_len: Optional[int]   # fixed length, or None for the ragged draw below
    ragged: Optional[tuple] = None   # (lo, hi) inclusive uniform draw of each length
    peaked_frac: float = 0.0
    peak_factor: float = 8.0

    @property
    def G(self) -> int:
        return self.h_q // self.h_kv

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def seed(self) -> int:
        return 1000 + self.cfg

    def seq_lens(self) -> np.ndarray:
        if self.ragged is None:
            return np.full(self.batch, self.seq_len, dtype=np.int32)
        rng = np.random.Generator(np.random.PCG64(_child(self.seed, 3)))
        lo, hi = self.ragged
        return rng.integers(lo, hi, size=self.batch, endpoint=True).astype(np.int32)

    def kv_bytes(self, seq_lens: Optional[np.ndarray] = None) -> int:
        """Bytes of K plus V read once (the algorithmic HBM traffic)."""
        sl = self.seq_lens() if seq_lens is None else seq_lens
        esize = 4 if self.dtype == "f32" else 2
        return int(np.clip(sl, 0, None).sum()) * self.h_kv * self.d * esize * 2


WORKLOADS = {
    1: Workload(1, "tiny_fp32_G8_d64_S256", "f32", 1, 8, 1, 64, 256),
    2: Workload(2, "8b_shaped_hq32_hkv8_d128_S8192", "bf16", 1, 32, 8, 128, 8192),
    3: Workload(3, "single_kv_group_hq8_hkv1_d128_S32768", "bf16", 1, 8, 1, 128, 32768),
    4: Workload(4, "70b_shaped_ragged_b64_hq64_hkv8_d128_S1k-32k", "bf16", 64, 64, 8, 128, None,
                ragged=(1024, 32768)),
    5: Workload(5, "stress_b8_hq64_hkv8_d128_S131072_peaked", "bf16", 8, 64, 8, 128, 131072,
                peaked_frac=0.001, peak_factor=8.0),
}


def _child(seed: int, idx: int) -> np.random.SeedSequence:
    """Child stream idx of a seed: 0 q, 1 k, 2 v, 3 seq_lens, 4 peaked rows."""
    return np.random.SeedSequence(seed).spawn(5)[idx]


# --------------------------------------------------------------------------------------
# bf16 bit handling (input preparation only)
# --------------------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16, nearest-even, returning the raw 16 bits as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 22
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        flat_o[s:s + step] = ((c + (((c >> 16) & 1) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------
# Host generation (numpy)
# --------------------------------------------------------------------------------------


@dataclass
class HostCase:
    q: np.ndarray            # uint16 bf16 bits, float16 or float32, [batch, (t_q,) h_q, d]
    k: np.ndarray            # [sum(seq_lens), h_kv, d]
    v: np.ndarray
    seq_lens: np.ndarray     # int32[batch]
    scale: float
    dtype: str
    peaked_rows: List[np.ndarray] = field(default_factory=list)


def _normal(seed: int, idx: int, n: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(_child(seed, idx)))
    return rng.standard_normal(n, dtype=np.float32)


def host_case(batch: int, h_q: int, h_kv: int, d: int, seq_lens: Sequence[int], dtype: str = "bf16",
              seed: int = 0, scale: Optional[float] = None, peaked_frac: float = 0.0,
              peak_factor: float = 8.0, t_q: int = 0) -> HostCase:
    """Draw q, k, v for the given shape on the host; t_q > 0 gives q t_q query
    tokens per sequence ([batch, t_q, h_q, d])."""
    sl = np.asarray(seq_lens, dtype=np.int32).reshape(batch)
    rows = int(np.clip(sl, 0, None).sum())
    qshape = (batch, t_q, h_q, d) if t_q > 0 else (batch, h_q, d)
    q = _normal(seed, 0, int(np.prod(qshape))).reshape(qshape)
    k = _normal(seed, 1, rows * h_kv * d).reshape(rows, h_kv, d)
    v = _normal(seed, 2, rows * h_kv * d).reshape(rows, h_kv, d)
    peaks: List[np.ndarray] = []
    if peaked_frac > 0.0:
        rng = np.random.Generator(np.random.PCG64(_child(seed, 4)))
        base = 0
        for S in np.clip(sl, 0, None):
            n = int(np.floor(peaked_frac * S))
            idx = np.sort(rng.choice(int(S), size=n, replace=False)) if n else np.zeros(0, np.int64)
            k[base + idx] *= np.float32(peak_factor)
            peaks.append(idx)
            base += int(S)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    elif dtype == "f16":
        q, k, v = q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)   # nearest even
    elif dtype != "f32":
        raise ValueError(dtype)
    return HostCase(q, k, v, sl, float(scale), dtype, peaks)


def host_prefill_case(batch: int, h_q: int, h_kv: int, d: int, seq_lens: Sequence[int], dtype: str = "bf16",
                      seed: int = 0, scale: Optional[float] = None, peaked_frac: float = 0.0,
                      peak_factor: float = 8.0) -> HostCase:
    """Prefill inputs: q [sum(seq_lens), h_q, d] (every token a query), k and v as
    host_case draws them (same streams and peaked rows)."""
    c = host_case(batch, h_q, h_kv, d, seq_lens, dtype, seed=seed, scale=scale, peaked_frac=peaked_frac,
                  peak_factor=peak_factor)
    rows = int(np.clip(c.seq_lens, 0, None).sum())
    qf = _normal(seed, 0, rows * h_q * d).reshape(rows, h_q, d)
    if dtype == "bf16":
        qf = f32_to_bf16_bits(qf)
    elif dtype == "f16":
        qf = qf.astype(np.float16)
    c.q = qf
    return c


# Causal prefill of one KV group over a 32K-token sequence (the long-context
# prefill panel: T_q = S_kv = 32768, h_q 8, h_kv 1, d_head 128, bf16).
PREFILL_32K = Workload(6, "prefill_single_kv_group_hq8_hkv1_d128_S32768", "bf16", 1, 8, 1, 128, 32768)


def host_workload(w: Workload) -> HostCase:
    return host_case(w.batch, w.h_q, w.h_kv, w.d, w.seq_lens(), w.dtype, seed=w.seed,
                     scale=w.scale, peaked_frac=w.peaked_frac, peak_factor=w.peak_factor)


# --------------------------------------------------------------------------------------
# Device generation (torch); imported lazily so the CPU-only paths need no torch device
# --------------------------------------------------------------------------------------


@dataclass
class DeviceCase:
    q: "object"              # torch tensors on the device
    k: "object"
    v: "object"
    seq_lens: "object"       # int32 device tensor
    seq_lens_host: np.ndarray
    scale: float
    dtype: str


def _torch_normal(shape, seed: int, device, out_dtype, chunk_rows: int = 1 << 18):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=out_dtype, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        blk = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        flat[r0:r1].copy_(blk)   # float32 -> bf16 copy rounds to nearest even
    return out


def device_case(batch: int, h_q: int, h_kv: int, d: int, seq_lens: Sequence[int], dtype: str = "bf16",
                seed: int = 0, scale: Optional[float] = None, peaked_frac: float = 0.0,
                peak_factor: float = 8.0, device: str = "cuda", t_q: int = 0) -> DeviceCase:
    """Draw q, k, v directly on the device (for multi-GiB workloads)."""
    import torch
    sl = np.asarray(seq_lens, dtype=np.int32).reshape(batch)
    rows = int(np.clip(sl, 0, None).sum())
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    base_seed = int(np.random.SeedSequence(seed).generate_state(1)[0])
    qshape = (batch, t_q, h_q, d) if t_q > 0 else (batch, h_q, d)
    q = _torch_normal(qshape, base_seed + 0, device, tdt)
    k = _torch_normal((rows, h_kv, d), base_seed + 1, device, tdt)
    v = _torch_normal((rows, h_kv, d), base_seed + 2, device, tdt)
    if peaked_frac > 0.0:
        g = torch.Generator(device=device)
        g.manual_seed(base_seed + 4)
        base = 0
        for S in np.clip(sl, 0, None):
            n = int(np.floor(peaked_frac * int(S)))
            if n:
                idx = torch.randperm(int(S), generator=g, device=device)[:n] + base
                k[idx] = (k[idx].float() * float(peak_factor)).to(tdt)
            base += int(S)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    sl_dev = torch.from_numpy(sl.copy()).to(device)
    return DeviceCase(q, k, v, sl_dev, sl, float(scale), dtype)


def device_queries(batch: int, t_q: int, h_q: int, d: int, dtype: str = "bf16", seed: int = 0,
                   device: str = "cuda"):
    """A seeded N(0,1) query block [batch, t_q, h_q, d] drawn on the device."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    base_seed = int(np.random.SeedSequence(seed).generate_state(1)[0])
    return _torch_normal((batch, t_q, h_q, d), base_seed, device, tdt)


def device_prefill_case(batch: int, h_q: int, h_kv: int, d: int, seq_lens: Sequence[int], dtype: str = "bf16",
                        seed: int = 0, scale: Optional[float] = None, device: str = "cuda") -> DeviceCase:
    """Prefill inputs drawn on the device: q [sum(seq_lens), h_q, d], k and v
    [sum(seq_lens), h_kv, d]."""
    import torch
    sl = np.asarray(seq_lens, dtype=np.int32).reshape(batch)
    rows = int(np.clip(sl, 0, None).sum())
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    base_seed = int(np.random.SeedSequence(seed).generate_state(1)[0])
    q = _torch_normal((rows, h_q, d), base_seed + 0, device, tdt)
    k = _torch_normal((rows, h_kv, d), base_seed + 1, device, tdt)
    v = _torch_normal((rows, h_kv, d), base_seed + 2, device, tdt)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    return DeviceCase(q, k, v, torch.from_numpy(sl.copy()).to(device), sl, float(scale), dtype)


def device_workload(w: Workload, device: str = "cuda") -> DeviceCase:
    return device_case(w.batch, w.h_q, w.h_kv, w.d, w.seq_lens(), w.dtype, seed=w.seed,
                       scale=w.scale, peaked_frac=w.peaked_frac, peak_factor=w.peak_factor,
                       device=device)


def to_host_bits(t) -> np.ndarray:
    """A device bf16/fp32 tensor as the host array the oracle reads (uint16 bits or float32)."""
    import torch
    c = t.detach().contiguous().cpu()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    if c.dtype in (torch.float32, torch.float16):
        return c.numpy()
    raise TypeError(c.dtype)


def from_host_bits(a: np.ndarray, device: str = "cuda"):
    """A host uint16 (bf16 bits) or float32 array as a device tensor."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype in (np.float32, np.float16):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    raise TypeError(a.dtype)
