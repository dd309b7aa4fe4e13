"""split_kv_decode_noalloc against split_kv_decode, through the C ABI.

The no-allocation entry point runs the same kernels with the key-split
partials in the library's static scratch array instead of a caller
workspace, so its per-shard partials must equal split_kv_decode's bit for
bit.  Two calls in a row, the second with a smaller input (fewer shards,
requests and heads, a shorter context and a different split count), check
that nothing the first call left in the array leaks into the second; both
are also compared with the oracle at the bf16 tolerances."""

import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import tensor, host64, compare, say, BF16_O, BF16_LSE

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    import ring_attention_02_amd as ra
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return ra


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _case(ra, cfg, n_shards, B, hq, hkv, t_shard, lens):
    d = 128
    lib = ra.lib()
    ws = lib.split_kv_decode_workspace(n_shards, B, hq, hkv, d, t_shard)
    assert ws > 0, "the case must use key splits (the scratch array)"
    say(f"no-alloc decode: shards={n_shards} B={B} hq={hq} hkv={hkv} t_shard={t_shard} workspace={ws} B")
    q, q64 = tensor(cfg, 1, 0, (B, hq, d), torch.bfloat16)
    ks, k64 = tensor(cfg, 2, 0, (n_shards, B, t_shard, hkv, d), torch.bfloat16)
    vs, v64 = tensor(cfg, 3, 0, (n_shards, B, t_shard, hkv, d), torch.bfloat16)
    lens_t = torch.from_numpy(np.asarray(lens, dtype=np.int64).reshape(n_shards, B)).cuda()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    scale = ctypes.c_float(1.0 / np.sqrt(d))
    outs = []
    for noalloc in (False, True):
        o = torch.full((n_shards, B, hq, d), 9.0, device="cuda")
        lse = torch.full((n_shards, B, hq), 9.0, device="cuda")
        if noalloc:
            st = lib.split_kv_decode_noalloc(_ptr(q), _ptr(ks), _ptr(vs), ra.CP_BF16, n_shards, B, t_shard,
                                             _ptr(lens_t), hq, hkv, d, d, scale, _ptr(o), _ptr(lse), stream)
        else:
            w = torch.empty(ws, dtype=torch.uint8, device="cuda")
            st = lib.split_kv_decode(_ptr(q), _ptr(ks), _ptr(vs), ra.CP_BF16, n_shards, B, t_shard,
                                     _ptr(lens_t), hq, hkv, d, d, scale, _ptr(o), _ptr(lse), _ptr(w),
                                     ctypes.c_size_t(ws), stream)
        assert st == ra.CP_OK, ra.last_error()
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o_a, l_a), (o_b, l_b) = outs
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b), "no-alloc partials differ from split_kv_decode's"
    lens_np = np.asarray(lens, dtype=np.int64).reshape(n_shards, B)
    for b in range(B):
        for s in range(n_shards):
            n = int(lens_np[s, b])
            if n == 0:
                ro, rl = np.zeros((1, hq, d)), np.full((1, hq), -np.inf)
            else:
                ro, rl = oracle.attention_ref(q64[b:b + 1, None], k64[s, b:b + 1, :n], v64[s, b:b + 1, :n])
                ro, rl = ro[:, 0], rl[:, 0]
            compare(host64(o_b[s, b:b + 1]), host64(l_b[s, b:b + 1]), ro, rl, BF16_O, BF16_LSE,
                    f"shard {s} request {b}")


def test_noalloc_decode_matches_workspace_decode_twice(ra):
    # first call: 4 shards x 2 requests x 2 kv heads = 16 work items (32 splits)
    _case(ra, 601, 4, 2, 16, 2, 8192, [8192, 5000, 1, 0, 8000, 8192, 333, 7777])
    # second call, smaller: 2 shards x 1 request x 1 kv head, 3000 slots (11 splits)
    _case(ra, 602, 2, 1, 8, 1, 3000, [3000, 1234])


def test_noalloc_rejects_bad_arguments(ra):
    lib = ra.lib()
    fake = ctypes.c_void_p(1 << 20)
    st = lib.split_kv_decode_noalloc(fake, fake, fake, ra.CP_BF16, 1, 1, 64, None, 64, 2, 128, 128,
                                     ctypes.c_float(0.1), fake, fake, None)
    assert st == ra.CP_EUNSUPPORTED            # 32 query heads per kv head
    st = lib.split_kv_decode_noalloc(fake, fake, fake, ra.CP_BF16, 1, 1, 64, None, 8, 1, 128, 128,
                                     ctypes.c_float(-1.0), fake, fake, None)
    assert st == ra.CP_EINVAL
