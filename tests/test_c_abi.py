"""The C ABI from plain C: tests/c_abi_host.c includes nothing but
include/ringattn.h, links the shared library and calls the host entry points
(partition, slot mapping with and without a block table, ring schedule,
classification, KV reorganisation index, an error path).  It is compiled as
strict C11 with warnings as errors, run, and every printed result is
compared with the oracle."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "ring_attention_02_amd")


def _run_program(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "c_abi_host")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_host.c"), "-L", PKG, "-lringattn", f"-Wl,-rpath,{PKG}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    return res.stdout.splitlines()


def test_c_program_calls_the_host_entry_points(tmp_path):
    lines = _run_program(tmp_path)
    vals = {}
    partitions = {}
    rank = None
    for ln in lines:
        name, *rest = ln.split()
        if name == "partition_rank":
            rank = int(rest[0])
        elif name in ("local", "restore"):
            partitions.setdefault(rank, {})[name] = [int(x) for x in rest]
        else:
            vals[name] = rest

    import ring_attention_02_amd as ra
    assert int(vals["abi"][0]) == ra.lib().cp_abi_version()

    lens = [10, 7]
    ref_local, ref_restore = oracle.partition_ref(lens, 2)
    for r in range(2):
        assert partitions[r]["local"] == list(ref_local[r])
        assert partitions[r]["restore"] == list(ref_restore)

    pos = 3 * np.arange(40) + 1
    dev, slot = oracle.slot_mapping_ref(pos, 8, 2, 2, 2)
    assert [int(x) for x in vals["dev"]] == list(dev) and [int(x) for x in vals["slot"]] == list(slot)
    table = np.array([4, 0, 3, 1, 2], dtype=np.int32)
    dev, slot = oracle.slot_mapping_ref(pos, 8, 2, 2, 2, block_table=table)
    assert [int(x) for x in vals["dev_table"]] == list(dev)
    assert [int(x) for x in vals["slot_table"]] == list(slot)

    assert [int(x) for x in vals["ring_src"]] == oracle.ring_schedule_ref(2, 4)
    parts = [int(x) for x in vals["ring_parts"]]
    assert list(zip(parts[0::2], parts[1::2])) == oracle.zigzag_ring_chunks_ref(2, 4)

    assert [int(x) for x in vals["classify"]] == [oracle.classify_ref(100, 50, 0, 64, True),
                                                  oracle.classify_ref(100, 50, 120, 10, True),
                                                  oracle.classify_ref(100, 50, 150, 10, True)]
    assert [int(x) for x in vals["classify"]] == [oracle.FULL, oracle.DIAG, oracle.SKIP]

    src, dev_lens = oracle.reorg_index_ref(lens, 4, 2, 2, 1)
    assert [int(x) for x in vals["reorg_src"]] == list(src)
    assert [int(x) for x in vals["reorg_dev_lens"]] == list(np.asarray(dev_lens).ravel())

    assert vals["status_string"][0].startswith("CP_EINVAL")


@pytest.mark.gpu
def test_c_program_runs_two_ring_steps_on_the_device(tmp_path):
    """tests/c_abi_device.c: device memory from the HIP runtime, two
    ring_attn_step calls (a FULL block, then a diagonal block merged in with
    accumulate), no framework anywhere; the result against the oracle over
    both blocks' keys."""
    import seeded_inputs as si
    from gpu_util import compare, say, BF16_O, BF16_LSE
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "c_abi_device")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_device.c"), "-L", PKG, "-lringattn", f"-Wl,-rpath,{PKG}",
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lm", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    sq, ska, skb, hq, hkv, d = 200, 300, 150, 8, 2, 128
    q_pos0, ka_pos0, kb_pos0 = 400, 0, 300
    cfg = 61
    q = si.normal_bf16_bits(cfg, 1, 0, (sq, hq, d))
    ka = si.normal_bf16_bits(cfg, 2, 0, (ska, hkv, d))
    va = si.normal_bf16_bits(cfg, 3, 0, (ska, hkv, d))
    kb = si.normal_bf16_bits(cfg, 2, 1, (skb, hkv, d))
    vb = si.normal_bf16_bits(cfg, 3, 1, (skb, hkv, d))
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        np.array([sq, ska, skb, hq, hkv, d, q_pos0, ka_pos0, kb_pos0, 1], dtype="<i8").tofile(f)
        for a in (q, ka, va, kb, vb):
            np.ascontiguousarray(a, dtype="<u2").tofile(f)
    say(f"C program: two ring steps sq={sq} sk={ska}+{skb} hq={hq} hkv={hkv} d={d}")
    res = subprocess.run([exe, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = np.fromfile(outp, dtype=np.uint8)
    o = raw[:4 * sq * hq * d].view("<f4").reshape(1, sq, hq, d)
    lse = raw[4 * sq * hq * d:4 * sq * hq * (d + 1)].view("<f4").reshape(1, sq, hq)
    cls = raw[4 * sq * hq * (d + 1):].view("<i4")
    assert cls.tolist() == [oracle.classify_ref(q_pos0, sq, ka_pos0, ska, True),
                            oracle.classify_ref(q_pos0, sq, kb_pos0, skb, True)] == [oracle.FULL, oracle.DIAG]
    f64 = lambda bits: si.bf16_bits_to_f32(bits).astype(np.float64)[None]
    k_all = np.concatenate([f64(ka), f64(kb)], 1)
    v_all = np.concatenate([f64(va), f64(vb)], 1)
    k_pos = np.concatenate([ka_pos0 + np.arange(ska), kb_pos0 + np.arange(skb)])
    o_ref, lse_ref = oracle.attention_ref(f64(q), k_all, v_all, q_pos0 + np.arange(sq), k_pos, True)
    compare(o, lse, o_ref, lse_ref, BF16_O, BF16_LSE, "C program, two ring steps")
