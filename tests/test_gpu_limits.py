"""GPU parity at the per-launch limits of the boundary.

* ring_attn_step_jobs with every slot in use: 4 query chunks, each over 4
  K/V segments of ragged lengths at their own positions (FULL, diagonal and
  invisible ones, accumulate on some jobs), and 4 forwarded ranges, on a
  small grid (8-wave key-split workgroups) and on a grid large enough for
  256-row workgroups (sampled heads).
* lse_merge at its largest head dimension (512) over 16 parts, and at the
  smallest (4) with bf16 output.
* One K/V segment of more than a million keys (2 GiB per tensor): the tile
  descriptors are re-based every 2^30 bytes, and with a ragged end every tile
  gets its own descriptor at offsets past 2^31, in the 8-wave, the 8-wave
  with backward (odd-round) sweeps and the 256-row forms (sampled rows).

Every result is compared element by element with the oracle."""

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


# Each job: (q_pos0, accumulate, [(segment length, k_pos0)] x 4).  The
# segments of a job are visible to its queries in different ways: wholly
# earlier (FULL), crossing the queries' positions (diagonal), or later
# than every query (invisible, skipped on the host).
JOBS = [
    (2000, False, [(70, 0), (129, 1950), (64, 500), (200, 9000)]),
    (300, True, [(201, 100), (64, 0), (33, 350), (150, 600)]),
    (5000, False, [(257, 4800), (1, 10), (190, 1200), (96, 4999)]),
    (0, True, [(65, 0), (130, 100), (64, 64), (17, 7)]),
]


@pytest.mark.parametrize("sq,hq,hkv,sampled", [(150, 4, 2, None), (300, 64, 8, [0, 9, 31, 63])])
def test_jobs_with_every_slot_in_use(ra, sq, hq, hkv, sampled):
    dqk = dv = 128
    say(f"jobs at the limits: 4 jobs x 4 segments, 4 forwards, sq={sq} hq={hq} hkv={hkv}")
    heads = list(range(hq)) if sampled is None else sampled
    jobs, refs = [], []
    for i, (q0, acc, segs) in enumerate(JOBS):
        cfg = 500 + 10 * i
        q, q64 = tensor(cfg, 1, 0, (1, sq, hq, dqk), torch.bfloat16)
        o = torch.full((1, sq, hq, dv), 3.0, device="cuda")
        lse = torch.full((1, sq, hq), 1.0, device="cuda")
        ks, vs, kp, seg_args = [], [], [], []
        if acc:   # an earlier partial over 50 keys just before the queries
            k2, k2_64 = tensor(cfg, 2, 9, (1, 50, hkv, dqk), torch.bfloat16)
            v2, v2_64 = tensor(cfg, 3, 9, (1, 50, hkv, dv), torch.bfloat16)
            ra.ring_attn_step(q, k2, v2, o, lse, q_pos0=q0, k_pos0=max(0, q0 - 50), causal=True)
            ks, vs, kp = [k2_64], [v2_64], [max(0, q0 - 50) + np.arange(50)]
        for j, (n, p0) in enumerate(segs):
            k, k64 = tensor(cfg, 2, j, (1, n, hkv, dqk), torch.bfloat16)
            v, v64 = tensor(cfg, 3, j, (1, n, hkv, dv), torch.bfloat16)
            seg_args.append((k, v, p0))
            ks.append(k64)
            vs.append(v64)
            kp.append(p0 + np.arange(n))
        jobs.append(dict(q=q, o=o, lse=lse, q_pos0=q0, accumulate=acc, segments=seg_args))
        k_all, v_all, p_all = np.concatenate(ks, 1), np.concatenate(vs, 1), np.concatenate(kp)
        grp = hq // hkv
        ro = np.zeros((1, sq, len(heads), dv))
        rl = np.zeros((1, sq, len(heads)))
        for n_h, h in enumerate(heads):
            a, b = oracle.attention_ref(q64[:, :, [h]], k_all[:, :, [h // grp]], v_all[:, :, [h // grp]],
                                        q0 + np.arange(sq), p_all, True)
            ro[:, :, n_h], rl[:, :, n_h] = a[:, :, 0], b[:, :, 0]
        refs.append((o, lse, ro, rl))
    src = [torch.randn(n, device="cuda") for n in (8196, 4, 65540, 40)]
    dst = [torch.full_like(x, -1.0) for x in src]
    ra.ring_attn_step_jobs(jobs, causal=True, forward=list(zip(dst, src)))
    torch.cuda.synchronize()
    for i, (o, lse, ro, rl) in enumerate(refs):
        compare(host64(o[:, :, heads]), host64(lse[:, :, heads]), ro, rl, BF16_O, BF16_LSE, f"job {i}")
    for d, s_ in zip(dst, src):
        assert torch.equal(d, s_)


@pytest.mark.parametrize("n,rows,dv,out_bf16", [(16, 300, 512, False), (2, 1001, 4, True)])
def test_lse_merge_at_its_head_dim_limits(ra, n, rows, dv, out_bf16):
    say(f"lse_merge limits n={n} rows={rows} dv={dv} bf16={out_bf16}")
    r = np.random.default_rng(7 * n + dv)
    o_parts = r.standard_normal((n, rows, dv)).astype(np.float32)
    lse_parts = (r.standard_normal((n, rows)) * 4).astype(np.float32)
    lse_parts[:, :3] = -np.inf
    o_parts[:, :3] = 0.0
    lse_parts[n - 1, 3:40] = -np.inf              # one part empty on some rows
    o_parts[n - 1, 3:40] = 0.0
    o_ref, lse_ref = oracle.lse_merge_ref(list(o_parts.astype(np.float64)),
                                          list(lse_parts.astype(np.float64)))
    od, ld = ra.lse_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda(),
                          out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    o_gpu = host64(od)
    compare(o_gpu, host64(ld), o_ref, lse_ref, BF16_O if out_bf16 else 1e-5, 1e-5, "lse_merge")
    if out_bf16:
        # bf16 output: round-to-nearest-even leaves at most half an ulp, i.e.
        # 2^-8 of the value, on top of the float32 merge
        assert np.all(np.abs(o_gpu - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + 1e-5)


# (sk, sq, hq): queries at the end of the sequence see every key (causal)
HUGE = [
    (1 << 20, 64, 8),            # whole tiles: 8-wave, one round
    ((1 << 20) + 37, 64, 8),     # ragged end: a descriptor per tile, offsets past 2^31
    ((1 << 20) + 37, 640, 64),   # 8-wave, 320 workgroups: odd rounds sweep backwards
    (1 << 20, 1024, 128),        # 256-row workgroups (512 of them)
]


@pytest.mark.parametrize("idx", range(len(HUGE)))
def test_segment_of_more_than_2_gib(ra, idx):
    import seeded_inputs as si
    sk, sq, hq = HUGE[idx]
    hkv, d = 8, 128
    say(f"huge segment case {idx}: sk={sk} sq={sq} hq={hq} hkv={hkv} d={d}")
    k = si.device_normal(600, 2, idx, (1, sk, hkv, d), torch.bfloat16, "cuda")
    v = si.device_normal(600, 3, idx, (1, sk, hkv, d), torch.bfloat16, "cuda")
    q = si.device_normal(600, 1, idx, (1, sq, hq, d), torch.bfloat16, "cuda")
    q0 = sk - sq
    o = torch.empty((1, sq, hq, d), device="cuda")
    lse = torch.empty((1, sq, hq), device="cuda")
    ra.ring_attn_step(q, k, v, o, lse, q_pos0=q0, k_pos0=0, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    group = hq // hkv
    rows = [(t, h) for t in sorted({0, 1, sq // 2, sq - 1}) for h in sorted({0, hq - 1, hq // 2 + 1})]
    for kvh in sorted({h // group for _, h in rows}):
        sel = [(t, h) for t, h in rows if h // group == kvh]
        tt = np.array([t for t, _ in sel])
        hh = np.array([h for _, h in sel])
        k64, v64 = host64(k[0, :, kvh]), host64(v[0, :, kvh])
        q64 = host64(q[0][torch.from_numpy(tt).cuda(), torch.from_numpy(hh).cuda()])
        ro, rl = oracle.attention_ref(q64[None, :, None, :], k64[None, :, None, :], v64[None, :, None, :],
                                      q0 + tt, np.arange(sk), causal=True)
        o_s = host64(o[0][torch.from_numpy(tt).cuda(), torch.from_numpy(hh).cuda()])
        l_s = host64(lse[0][torch.from_numpy(tt).cuda(), torch.from_numpy(hh).cuda()])
        compare(o_s, l_s, ro[0, :, 0], rl[0, :, 0], BF16_O, BF16_LSE, f"huge {idx} kv head {kvh}")
        del k64, v64
    del k, v, q, o, lse
    torch.cuda.empty_cache()
