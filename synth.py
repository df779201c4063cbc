"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and places them in the storage layouts; it
holds none of the method's arithmetic (no dequantization, no dot products, no
activation quantization).  Both the CPU oracle and the HIP library consume its
outputs; neither is imported here.

The pages' workloads are DeepSeek-V4-Flash GGUF tensors that are not available;
these generators stand in for them with the shapes and value distributions the
workload definitions below state:

  * Q8_0 weights: int8 quants uniform in [-127, 127], one fp16 scale per
    32-block drawn uniform [1e-3, 1e-2] and rounded to fp16 (nearest even).
  * Q4_K-style weights: 4-bit quants uniform 0..15, 6-bit sub-scales and
    sub-mins uniform 0..63, fp16 d and dmin uniform [1e-4, 1e-2].  Uniform
    random bytes give exactly these distributions for the nibbles and for the
    sixteen 6-bit fields of the 96-bit scale string, so the packed bytes are
    drawn directly.
  * activations fp32 N(0, 1); prefill activations bf16 = N(0, 1) rounded to
    nearest even.
  * routed MoE: per token, top-6 experts uniformly without replacement (first 6
    of a seeded permutation) or by Zipf(1.1) popularity (Gumbel-top-k over
    log p_i with p_i proportional to (i+1)^-1.1); routing weights from N(0, 1)
    logits through a sigmoid, normalized to sum 1 over the token's experts.
"""
from __future__ import annotations

import numpy as np

Q8_0_BLOCK_BYTES = 34   # fp16 scale + 32 int8
Q4K_BLOCK_BYTES = 144   # fp16 d, fp16 dmin, 12 bytes of 6-bit fields, 128 bytes of nibbles


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _fp16_uniform(g: np.random.Generator, lo: float, hi: float, size) -> np.ndarray:
    return g.uniform(lo, hi, size=size).astype(np.float16)


def q8_0_weight(g: np.random.Generator, N: int, K: int, d_lo: float = 1e-3, d_hi: float = 1e-2) -> np.ndarray:
    """[N, K/32*34] uint8, rows of Q8_0 blocks (scale bytes first)."""
    assert K % 32 == 0
    nb = K // 32
    d = _fp16_uniform(g, d_lo, d_hi, (N, nb))
    q = g.integers(-127, 128, size=(N, nb, 32), dtype=np.int16).astype(np.int8)
    blocks = np.empty((N, nb, Q8_0_BLOCK_BYTES), np.uint8)
    blocks[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
    blocks[:, :, 2:] = q.view(np.uint8)
    return blocks.reshape(N, nb * Q8_0_BLOCK_BYTES)


def q8_0_from_parts(d_fp16: np.ndarray, q_int8: np.ndarray) -> np.ndarray:
    """Place given scales [N, nb] (float16) and quants [N, nb, 32] (int8) into Q8_0 rows."""
    d_fp16 = np.asarray(d_fp16, np.float16)
    q_int8 = np.asarray(q_int8, np.int8)
    N, nb = d_fp16.shape
    blocks = np.empty((N, nb, Q8_0_BLOCK_BYTES), np.uint8)
    blocks[:, :, 0:2] = d_fp16.view(np.uint8).reshape(N, nb, 2)
    blocks[:, :, 2:] = q_int8.view(np.uint8)
    return blocks.reshape(N, nb * Q8_0_BLOCK_BYTES)


def q4k_weight(g: np.random.Generator, N: int, K: int, lo: float = 1e-4, hi: float = 1e-2) -> np.ndarray:
    """[N, K/256*144] uint8, rows of Q4_K-style superblocks."""
    assert K % 256 == 0
    ns = K // 256
    d = _fp16_uniform(g, lo, hi, (N, ns))
    dmin = _fp16_uniform(g, lo, hi, (N, ns))
    rest = g.integers(0, 256, size=(N, ns, Q4K_BLOCK_BYTES - 4), dtype=np.uint8)
    sb = np.empty((N, ns, Q4K_BLOCK_BYTES), np.uint8)
    sb[:, :, 0:2] = d.view(np.uint8).reshape(N, ns, 2)
    sb[:, :, 2:4] = dmin.view(np.uint8).reshape(N, ns, 2)
    sb[:, :, 4:] = rest
    return sb.reshape(N, ns * Q4K_BLOCK_BYTES)


# FP8 E4M3 (128 x 128 block scales) and FP4 E2M1 (1 x 32 scales) expert
# matrices, UE8M0 scales.  One buffer per matrix: the codes, then the scale
# bytes from the next multiple of 256 bytes, then zeros up to a multiple of 16
# bytes.
FMT_FP8_B128 = 2
FMT_FP4_MX = 3
E4M3_NAN_CODES = (0x7F, 0xFF)


def _align256(x: int) -> int:
    return (x + 255) // 256 * 256


def scaled_matrix_bytes(fmt: int, N: int, K: int) -> int:
    """Bytes of an FP8 / FP4 matrix buffer: codes, padding to 256, scales, padding to 16."""
    if fmt == FMT_FP8_B128:
        end = _align256(N * K) + (N + 127) // 128 * (K // 128)
    elif fmt == FMT_FP4_MX:
        end = _align256(N * K // 2) + N * (K // 32)
    else:
        raise ValueError(fmt)
    return (end + 15) // 16 * 16


def fp8_from_parts(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Place E4M3 codes uint8 [N, K] and UE8M0 scales uint8 [ceil(N/128), K/128] into one buffer."""
    N, K = codes.shape
    assert scales.shape == ((N + 127) // 128, K // 128)
    buf = np.zeros(scaled_matrix_bytes(FMT_FP8_B128, N, K), np.uint8)
    buf[:N * K] = codes.reshape(-1)
    buf[_align256(N * K):_align256(N * K) + scales.size] = scales.reshape(-1)
    return buf


def fp4_from_parts(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Place packed E2M1 codes uint8 [N, K/2] (element 2i in the low nibble of byte i) and
    UE8M0 scales uint8 [N, K/32] into one buffer."""
    N, half = codes.shape
    K = 2 * half
    assert scales.shape == (N, K // 32)
    buf = np.zeros(scaled_matrix_bytes(FMT_FP4_MX, N, K), np.uint8)
    buf[:N * half] = codes.reshape(-1)
    buf[_align256(N * half):_align256(N * half) + scales.size] = scales.reshape(-1)
    return buf


def fp8_weight(g: np.random.Generator, N: int, K: int, s_lo: int = 118, s_hi: int = 122) -> np.ndarray:
    """FP8 E4M3 matrix buffer: codes uniform over the 254 non-NaN codes, scales uniform
    integers in [s_lo, s_hi] (2^-9 .. 2^-5 for the defaults)."""
    assert K % 128 == 0
    valid = np.setdiff1d(np.arange(256), E4M3_NAN_CODES).astype(np.uint8)
    codes = valid[g.integers(0, valid.size, size=(N, K))]
    scales = g.integers(s_lo, s_hi + 1, size=((N + 127) // 128, K // 128)).astype(np.uint8)
    return fp8_from_parts(codes, scales)


def fp4_weight(g: np.random.Generator, N: int, K: int, s_lo: int = 120, s_hi: int = 124) -> np.ndarray:
    """FP4 E2M1 matrix buffer: uniform random nibbles (all 16 codes are values), scales
    uniform integers in [s_lo, s_hi]."""
    assert K % 32 == 0
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = g.integers(s_lo, s_hi + 1, size=(N, K // 32)).astype(np.uint8)
    return fp4_from_parts(codes, scales)


def weight(fmt: int, g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """A synthetic matrix of any format (0 Q8_0, 1 Q4_K, 2 FP8 E4M3 B128, 3 FP4 E2M1 MX)."""
    return [q8_0_weight, q4k_weight, fp8_weight, fp4_weight][fmt](g, N, K)


def activations(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """fp32 [M, K] drawn N(0, 1)."""
    return g.standard_normal((M, K), dtype=np.float64).astype(np.float32)


def bf16_activations(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """bf16 bit patterns (uint16 [M, K]) of N(0, 1) rounded to nearest even."""
    import torch
    x = torch.from_numpy(g.standard_normal((M, K), dtype=np.float64).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def moe_ids_uniform(g: np.random.Generator, T: int, E: int, topk: int) -> np.ndarray:
    """int32 [T, topk]: per token the first topk entries of a seeded permutation of E."""
    return np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32).reshape(T, topk)


def moe_ids_zipf(g: np.random.Generator, T: int, E: int, topk: int, s: float = 1.1) -> np.ndarray:
    """int32 [T, topk]: Zipf(s) popularity by expert id, top-k without replacement
    via Gumbel-top-k (argsort of log p + Gumbel noise, largest first)."""
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    out = np.empty((T, topk), np.int32)
    for t in range(T):
        key = logp + g.gumbel(size=E)
        out[t] = np.argsort(-key, kind="stable")[:topk]
    return out


def routing_weights(g: np.random.Generator, T: int, topk: int) -> np.ndarray:
    """fp32 [T, topk]: sigmoid of N(0, 1) logits, normalized per token (fp64, then rounded)."""
    logits = g.standard_normal((T, topk))
    s = 1.0 / (1.0 + np.exp(-logits))
    return (s / s.sum(axis=1, keepdims=True)).astype(np.float32)


def moe_experts(g: np.random.Generator, E: int, D: int, F: int, fmt: int = 1):
    """Lists (gate, up, down) of E matrices in format fmt (Q4_K by default): gate/up [F, D], down [D, F]."""
    gate, up, down = [], [], []
    for _ in range(E):
        gate.append(weight(fmt, g, F, D))
        up.append(weight(fmt, g, F, D))
        down.append(weight(fmt, g, D, F))
    return gate, up, down


# --------------------------------------------------------------------------
# Workload definitions (seeded).  Sizes as the workload statements give them.
# --------------------------------------------------------------------------

WORKLOADS = {
    # Q8_0 GEMV, batch 1, 512 x 1024
    "q8_0_512x1024": dict(fmt="q8_0", N=512, K=1024, M=1, seed=0),
    # Q8_0 output projection 8192 -> 4096, batch 1
    "q8_0_out_4096x8192": dict(fmt="q8_0", N=4096, K=8192, M=1, seed=1),
    # paired low-rank style: one 4096 activation, 4096->1024 and 4096->512
    "q8_0_pair_1024+512x4096": dict(fmt="q8_0", N1=1024, N2=512, K=4096, M=1, seed=1),
    # Q4_K dense projection 4096 -> 8192, batch 1 and prefill batch 512
    "q4k_8192x4096": dict(fmt="q4k", N=8192, K=4096, M=1, seed=2),
    "q4k_prefill_512x8192x4096": dict(fmt="q4k", N=8192, K=4096, M=512, seed=2),
    # the Q8_0 prefill product on the matrix cores: 512 tokens through 4096 -> 8192
    "q8_0_prefill_512x8192x4096": dict(fmt="q8_0", N=8192, K=4096, M=512, seed=10),
    # grouped low-rank attention output: 8 groups of 1024 x 4096 on their own input slices
    "q8_0_grouped_8x1024x4096": dict(fmt="q8_0", G=8, N=1024, K=4096, M=1, seed=5),
    # routed MoE, 256 experts, top-6, D=4096, F=2048, T=1 and T=8
    "moe_e256_t1": dict(E=256, D=4096, F=2048, topk=6, T=1, ids="uniform", seed=3),
    "moe_e256_t8": dict(E=256, D=4096, F=2048, topk=6, T=8, ids="uniform", seed=3),
    # batched decode sweep: Q8_0 4096 -> 16384 at M in {1,2,4,8,16,32}
    "q8_0_16384x4096": dict(fmt="q8_0", N=16384, K=4096, Ms=(1, 2, 4, 8, 16, 32), seed=4),
    # routed MoE with reuse: 384 experts, top-6, 64 tokens, Zipf(1.1)
    "moe_e384_t64_zipf": dict(E=384, D=4096, F=2048, topk=6, T=64, ids="zipf", seed=4),
    # the ATOM expert formats on the routed path, one token: FP8 E4M3 with
    # 128 x 128 block scales over 256 experts, FP4 E2M1 with 1 x 32 scales over 384
    "moe_fp8_e256_t1": dict(E=256, D=4096, F=2048, topk=6, T=1, ids="uniform", fmt=FMT_FP8_B128, seed=6),
    # the same formats as dense 4096 -> 16384 mat-vecs, batch 1
    "fp8_16384x4096": dict(fmt=FMT_FP8_B128, N=16384, K=4096, M=1, seed=8),
    "fp4_16384x4096": dict(fmt=FMT_FP4_MX, N=16384, K=4096, M=1, seed=9),
    "moe_fp4_e384_t1": dict(E=384, D=4096, F=2048, topk=6, T=1, ids="uniform", fmt=FMT_FP4_MX, seed=7),
}
