"""Seeded synthetic inputs shared by the tests, the bench and the smoke run.

This module only draws random numbers and rounds them to bf16; it holds
none of the attention, merge, partition or slot-mapping arithmetic, so it
can serve both the CPU oracle and the GPU path without coupling them.

Recipe: numpy ``Generator(PCG64(SeedSequence((cfg, tensor_id, chunk_id))))``
draws ``standard_normal`` in float32; bf16 tensors are those float32 values
rounded to nearest-even bf16.  ``tensor_id`` is 1 for Q, 2 for K, 3 for V
(other ids are free for test-specific draws), ``chunk_id`` names the
sequence chunk / shard / request so that every piece is reproducible on
its own.
"""

import numpy as np

Q_ID, K_ID, V_ID = 1, 2, 3


def rng(cfg, tensor_id, chunk_id=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence((cfg, tensor_id, chunk_id))))


def normal_f32(cfg, tensor_id, chunk_id, shape):
    """float32 N(0, 1) samples of `shape` for (cfg, tensor, chunk)."""
    return rng(cfg, tensor_id, chunk_id).standard_normal(shape, dtype=np.float32)


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite normal draws, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact float32 value of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def normal_bf16_bits(cfg, tensor_id, chunk_id, shape):
    """bf16 bit patterns of N(0, 1) draws (float32 draws rounded to bf16)."""
    return f32_to_bf16_bits(normal_f32(cfg, tensor_id, chunk_id, shape))


# The five workloads, as sizes only (the arithmetic lives in the oracle and
# in the HIP library, never here).
CONFIGS = {
    1: dict(name="tiny non-causal ring, fp32", batch=1, heads=4, d=64, seq=512,
            n_blocks=4, dtype="f32"),
    2: dict(name="zigzag causal prefill, rank 0 of cp=4, seq 8192", seq=8192, cp=4,
            rank=0, hq=32, hkv=32, d=128, dtype="bf16"),
    3: dict(name="GQA decode over 8 sequence shards, ctx 131072", batch=64, hq=64,
            hkv=8, d=128, ctx=131072, block_size=128, interleave=16, pcp=8, dcp=1,
            dtype="bf16"),
    4: dict(name="zigzag causal prefill, rank 0 of cp=8, seq 1048576", seq=1048576,
            cp=8, rank=0, hq=64, hkv=8, d=128, dtype="bf16"),
    5: dict(name="segmented chunked prefill, MLA shape", q_len=4096, q_pos0=131072,
            heads=128, d_qk=192, d_v=128, kv_len=135168, segment=8192, dtype="bf16"),
}


def device_seed(cfg, tensor_id, chunk_id=0):
    """63-bit seed for a device-side generator, from the same SeedSequence key."""
    state = np.random.SeedSequence((cfg, tensor_id, chunk_id)).generate_state(1, dtype=np.uint64)
    return int(state[0] & np.uint64((1 << 63) - 1))


def device_normal(cfg, tensor_id, chunk_id, shape, dtype, device):
    """N(0, 1) draws made on the GPU (for inputs too large to draw on the host).

    torch's device generator is seeded from (cfg, tensor, chunk); float32 draws
    are rounded to `dtype` (round-to-nearest-even for bf16).  The oracle reads
    back exactly the values the kernels receive, so both sides see the same
    inputs.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(cfg, tensor_id, chunk_id))
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    return x if dtype == torch.float32 else x.to(dtype)
