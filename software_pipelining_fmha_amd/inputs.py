"""Seeded synthetic inputs for the attention forward and backward passes.

This module is shared by the HIP path's callers (tests, bench) and by the CPU
oracle's callers. It draws numbers and picks rows. It holds no part of the
attention arithmetic.

Workloads. Each page evaluates FMHA forward in FP16 with batch 4, 32 heads and
head dim 128, at sequence lengths from 1K to 16K:
- Twill (OSDI'26), section 6.2 and Figures 7-8;
- Tawa (CGO'26), section V-D and Figure 10.
The pages measure no dataset. Inputs are i.i.d. N(0,1) draws rounded to fp16,
in the [B, H, N, d] layout.

Recipe, per workload index c:
- rng = numpy.random.default_rng(20260000 + c);
- draw Q, K, V in that order, each as float32 standard_normal of shape
  [B, H, N, d], then round once to float16 (round-to-nearest-even);
- the causal workload's K is fp16(3 * z), with the product taken in float32;
- scale = float32(1 / sqrt(d)).
FP8 inputs (FP8_WORKLOADS): the same float32 draws as the FP16 workload of
the same shape, each tensor quantized on its own to OCP FP8 E4M3 with
descale = float32(amax / 448) (amax over the whole tensor) and bytes =
e4m3(RNE(x / descale)), the division in float32. Tawa (CGO'26), section V-D,
measures FP8 attention at batch 4, head dim 128, L from 1K to 16K.
Backward pass: the output gradient dO of workload c is one more float32
standard_normal draw of the same shape, from
numpy.random.default_rng(20260000 + c + DOUT_SEED_OFFSET), rounded once to
float16. The pages give no backward workload, so it reuses the forward
shapes.
GEMM (the warp-specialised GEMM of the performance-model page): A [M][K]
and B [K][N] are float32 standard_normal draws, A first, from
numpy.random.default_rng(20260900 + c) for GEMM workload c (or the seed a
test passes), each rounded once to float16. The page measures
M, N, K in {256, 512, 1024} with T_M, T_N, T_K in {64, 128}; Tawa (CGO'26),
section V-D, measures FP16 GEMM at M = N = 8192 with K from 256 to 16384.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

SEED_BASE = 20260000
SAMPLE_SEED_XOR = 0x5EED
DOUT_SEED_OFFSET = 500


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    k_gain: float = 1.0       # K = fp16(k_gain * z)
    sampled_rows: int = 0     # 0: the oracle checks every row

    @property
    def flops(self) -> float:
        """Counted work: 4*B*H*N^2*d. Causal counts half of it."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    @property
    def scale(self) -> np.float32:
        return np.float32(1.0 / np.sqrt(np.float64(self.d)))


WORKLOADS = (
    Workload("tiny_b1h1n128d64", 1, 1, 128, 64, False),
    Workload("b4h32n1024d128", 4, 32, 1024, 128, False),
    Workload("b4h32n4096d128", 4, 32, 4096, 128, False, sampled_rows=256),
    Workload("b4h32n16384d128", 4, 32, 16384, 128, False, sampled_rows=256),
    Workload("causal_b4h32n8192d128_k3", 4, 32, 8192, 128, True, k_gain=3.0,
             sampled_rows=256),
)
HEADLINE = 3

FP8_WORKLOADS = (
    Workload("fp8_tiny_b1h1n128d128", 1, 1, 128, 128, False),
    Workload("fp8_b4h32n1024d128", 4, 32, 1024, 128, False),
    Workload("fp8_b4h32n4096d128", 4, 32, 4096, 128, False, sampled_rows=256),
    Workload("fp8_b4h32n16384d128", 4, 32, 16384, 128, False, sampled_rows=256),
    Workload("fp8_causal_b4h32n8192d128_k3", 4, 32, 8192, 128, True, k_gain=3.0,
             sampled_rows=256),
)
FP8_SEED_OFFSET = 700


def draw_qkv(B: int, H: int, N: int, d: int, seed: int, k_gain: float = 1.0):
    """Q, K, V as float16 arrays of shape [B,H,N,d], drawn in that order."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    out = []
    for name in ("q", "k", "v"):
        z = rng.standard_normal(size=shape, dtype=np.float32)
        if name == "k" and k_gain != 1.0:
            z *= np.float32(k_gain)
        out.append(z.astype(np.float16))
        del z
    return tuple(out)


def quantize_e4m3(x: np.ndarray):
    """(bytes uint8, descale float32): x ~= descale * e4m3(bytes), per tensor."""
    import torch

    amax = float(np.abs(x).max())
    descale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    y = (x.astype(np.float32) / descale).astype(np.float32)
    b = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(b), descale


def draw_qkv_fp8(B: int, H: int, N: int, d: int, seed: int, k_gain: float = 1.0):
    """FP8 Q, K, V: ((q8, k8, v8) uint8 arrays, (dq, dk, dv) descales). The
    float32 draws are those of draw_qkv with the same arguments."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    bytes_, scales = [], []
    for name in ("q", "k", "v"):
        z = rng.standard_normal(size=shape, dtype=np.float32)
        if name == "k" and k_gain != 1.0:
            z *= np.float32(k_gain)
        b, sc = quantize_e4m3(z)
        del z
        bytes_.append(b)
        scales.append(sc)
    return tuple(bytes_), tuple(scales)


def fp8_workload_inputs(index: int):
    """((q8, k8, v8), (dq, dk, dv), scale) for FP8_WORKLOADS[index]."""
    w = FP8_WORKLOADS[index]
    b, sc = draw_qkv_fp8(w.B, w.H, w.N, w.d, SEED_BASE + FP8_SEED_OFFSET + index, w.k_gain)
    return b, sc, w.scale


def fp8_workload_rows(index: int) -> np.ndarray:
    """The (b,h,i) triples the oracle checks for FP8_WORKLOADS[index]."""
    w = FP8_WORKLOADS[index]
    seed = (SEED_BASE + FP8_SEED_OFFSET + index) ^ SAMPLE_SEED_XOR
    if w.sampled_rows == 0:
        b, h, i = np.meshgrid(np.arange(w.B), np.arange(w.H), np.arange(w.N), indexing="ij")
        return np.stack([b.ravel(), h.ravel(), i.ravel()], 1).astype(np.int64)
    rows = sample_rows(w.B, w.H, w.N, w.sampled_rows, seed)
    if w.causal:
        extra = boundary_rows(w.B, w.H, w.N, 4, seed + 1)
        rows = np.unique(np.concatenate([rows, extra]), axis=0)
    return rows


def workload_inputs(index: int):
    """(q, k, v, scale) for WORKLOADS[index]."""
    w = WORKLOADS[index]
    q, k, v = draw_qkv(w.B, w.H, w.N, w.d, SEED_BASE + index, w.k_gain)
    return q, k, v, w.scale


def draw_dout(B: int, H: int, N: int, d: int, seed: int):
    """dO as a float16 array of shape [B,H,N,d]: one standard normal draw."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(size=(B, H, N, d), dtype=np.float32)
    return z.astype(np.float16)


def workload_dout(index: int):
    """The output gradient for WORKLOADS[index]."""
    w = WORKLOADS[index]
    return draw_dout(w.B, w.H, w.N, w.d, SEED_BASE + index + DOUT_SEED_OFFSET)


def sample_rows(B: int, H: int, N: int, n: int, seed: int) -> np.ndarray:
    """n distinct (b, h, i) triples, uniform over B*H*N, sorted by flat index."""
    rng = np.random.default_rng(seed)
    total = B * H * N
    n = min(n, total)
    flat = np.sort(rng.choice(total, size=n, replace=False))
    b, rem = np.divmod(flat, H * N)
    h, i = np.divmod(rem, N)
    return np.stack([b, h, i], axis=1).astype(np.int64)


# Row edges of the FP16 and FP8 forward kernels at head dim 128: a key tile
# (BN = 64) and a query tile (BM = 256) of a workgroup, plus the 32 query
# rows of one wave and the 128 rows of one group of four waves. The ABI
# reports BM and BN (fmha_query_tile, fmha_key_tile); a CPU test checks that
# they agree with these.
FWD_KEY_TILE = 64
FWD_QUERY_TILE = 256
TILE_EDGES = (32, FWD_KEY_TILE, 128, FWD_QUERY_TILE)


def boundary_rows(B: int, H: int, N: int, heads: int, seed: int,
                  tiles=TILE_EDGES) -> np.ndarray:
    """Rows at tile edges of a few seeded heads: 0, 1, t-1, t for each tile
    size t, and N-1."""
    rng = np.random.default_rng(seed)
    picks = rng.choice(B * H, size=min(heads, B * H), replace=False)
    idx = {0, 1, N - 1}
    for t in tiles:
        idx.update({t - 1, t})
    idx = sorted(i for i in idx if 0 <= i < N)
    rows = [(p // H, p % H, i) for p in sorted(picks) for i in idx]
    return np.asarray(rows, dtype=np.int64).reshape(-1, 3)


def workload_rows(index: int) -> np.ndarray:
    """The (b,h,i) triples the oracle checks for WORKLOADS[index]."""
    w = WORKLOADS[index]
    seed = (SEED_BASE + index) ^ SAMPLE_SEED_XOR
    if w.sampled_rows == 0:
        b, h, i = np.meshgrid(np.arange(w.B), np.arange(w.H), np.arange(w.N),
                              indexing="ij")
        return np.stack([b.ravel(), h.ravel(), i.ravel()], 1).astype(np.int64)
    rows = sample_rows(w.B, w.H, w.N, w.sampled_rows, seed)
    if w.causal:
        extra = boundary_rows(w.B, w.H, w.N, 4, seed + 1)
        rows = np.unique(np.concatenate([rows, extra]), axis=0)
    return rows


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


GEMM_SEED_BASE = 20260900


@dataclass(frozen=True)
class GemmWorkload:
    name: str
    M: int
    N: int
    K: int


GEMM_WORKLOADS = (
    GemmWorkload("gemm_m256n256k256", 256, 256, 256),
    GemmWorkload("gemm_m1024n1024k1024", 1024, 1024, 1024),
    GemmWorkload("gemm_m8192n8192k8192", 8192, 8192, 8192),
    GemmWorkload("gemm_m8192n8192k1024", 8192, 8192, 1024),
)
GEMM_HEADLINE = 2


def draw_gemm(M: int, N: int, K: int, seed: int):
    """A fp16 [M, K] and B fp16 [K, N], row-major."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)
    b = rng.standard_normal((K, N), dtype=np.float32).astype(np.float16)
    return a, b


def gemm_workload_inputs(index: int):
    w = GEMM_WORKLOADS[index]
    return draw_gemm(w.M, w.N, w.K, GEMM_SEED_BASE + index)


def gemm_sample_rows(M: int, tile_m: int, n: int, seed: int) -> np.ndarray:
    """Sorted distinct rows: the first and last row of every tile_m block
    (up to n of them), then seeded random rows up to n in total."""
    edges = sorted({r for t in range(0, M, tile_m) for r in (t, min(t + tile_m, M) - 1)})
    rows = set(edges[:n])
    rng = np.random.default_rng(seed ^ SAMPLE_SEED_XOR)
    while len(rows) < min(n, M):
        rows.add(int(rng.integers(0, M)))
    return np.array(sorted(rows), dtype=np.int64)
