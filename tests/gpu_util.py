"""Helpers shared by the GPU tests: device tensors from seeded inputs and
comparisons at the stated tolerances."""

import sys

import numpy as np

import seeded_inputs as si

# Tolerances (max abs error), from the workload statement.
F32_O = 1e-4
BF16_O = 2e-2
BF16_LSE = 1e-3
REL_L2 = 1e-2     # extra guard: ||O - O_ref|| / ||O_ref||


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def tensor(cfg, tid, chunk, shape, dtype):
    """Seeded host draw -> (device tensor, exact float64 values it holds)."""
    import torch
    if dtype == torch.float32:
        x = si.normal_f32(cfg, tid, chunk, shape)
        return torch.from_numpy(x).cuda(), x.astype(np.float64)
    bits = si.normal_bf16_bits(cfg, tid, chunk, shape)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return t, si.bf16_bits_to_f32(bits).astype(np.float64)


def host64(t):
    """Exact float64 copy of a device tensor (bf16 / float32 values are exact in float64)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def compare(o, lse, o_ref, lse_ref, o_tol, lse_tol, what=""):
    """Element-wise check of O and LSE against the oracle; -inf rows must match."""
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    fin_ref = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin_ref), f"{what}: -inf rows differ"
    assert np.all(np.isneginf(lse[~fin_ref])), f"{what}: empty rows must be -inf"
    assert np.all(o[~fin_ref] == 0.0), f"{what}: empty rows must have O = 0"
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse[fin_ref] - lse_ref[fin_ref]))) if fin_ref.any() else 0.0
    nrm = float(np.linalg.norm(o_ref))
    rel = float(np.linalg.norm(o - o_ref)) / nrm if nrm > 0 else 0.0
    say(f"  {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} relL2={rel:.3e}")
    assert err_o <= o_tol, f"{what}: O error {err_o} > {o_tol}"
    assert err_l <= lse_tol, f"{what}: LSE error {err_l} > {lse_tol}"
    if nrm > 0:
        assert rel <= REL_L2, f"{what}: relative L2 error {rel} > {REL_L2}"
    return err_o, err_l, rel


def whole_output_properties(o, lse, q, k, v, q_pos, k_pos0, group, scale, what):
    """Properties every row of a causal attention output must have, checked
    on the device over all rows (the sampled rows are checked exactly):

    * O and LSE are finite (every row sees at least one key);
    * O is a convex combination of the visible V rows, so each element lies
      within the column range of its kv head's V;
    * LSE = ln sum exp(s) is at least the score of any visible key: key 0 and
      the row's own position are visible to every row here;
    * LSE is at most the largest possible score (|q| max|k| scale) plus the
      log of the number of keys the row sees.

    o [S, H, dv] / lse [S, H] float32; q [S, H, d], k / v [Sk, Hkv, d] bf16 at
    absolute positions q_pos (device int64 [S]) and k_pos0 + arange(Sk)."""
    import torch
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), f"{what}: non-finite output"
    hkv = k.shape[1]
    vmin = v.float().amin(0).repeat_interleave(group, 0)          # [H, dv]
    vmax = v.float().amax(0).repeat_interleave(group, 0)
    slack = 1e-3
    assert bool((o >= vmin - slack).all()) and bool((o <= vmax + slack).all()), \
        f"{what}: O outside the range of V"
    for key_idx in (torch.zeros_like(q_pos), q_pos - k_pos0):
        kk = k[key_idx].float().repeat_interleave(group, 1)       # [S, H, d]
        chunk = 8192
        for a0 in range(0, q.shape[0], chunk):
            s_ = (q[a0:a0 + chunk].float() * kk[a0:a0 + chunk]).sum(-1) * scale
            assert bool((lse[a0:a0 + chunk] >= s_ - 1e-3).all()), f"{what}: LSE below a visible score"
        del kk
    qn = q.float().norm(dim=-1)                                   # [S, H]
    kmax = k.float().norm(dim=-1).amax(0).repeat_interleave(group, 0)   # [H]
    n_vis = (q_pos - k_pos0 + 1).double().log().float()[:, None]
    assert bool((lse <= qn * kmax * scale + n_vis + 1e-3).all()), f"{what}: LSE above its bound"
    say(f"  {what}: all {o.shape[0] * o.shape[1]} rows finite, within V's range and the LSE bounds")
