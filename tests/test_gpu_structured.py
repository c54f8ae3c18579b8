"""GPU parity of the structured lists (bsa_plan_structured) and their
attention through bsa_forward_csr: spatial and temporal heads of the Sparse
VideoGen page (section on its key idea), on the tile grid of the static
permutation.

* Row pointers and lists: bit-exact against the oracle's rule.
* Attention: the oracle's CSR attention on the same lists, with the
  forward's output and lse tolerances (small cases in full, the full-size
  grid on sampled (batch, head) slices and query tiles).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import DeviceRun, check_lse, check_output, to_bits

pytestmark = pytest.mark.gpu

W = S.Workload
CASES = [
    (W("st_small", 1, 2, 64, (8, 16, 16), 4, seed=31), [0, 1], 1, 1),
    (W("st_prefix", 2, 3, 128, (8, 8, 16), 4, seed=32, n_prefix=128), [1, 0, 1], 0, 2),
    (W("st_shape", 1, 2, 128, (16, 8, 8), 4, seed=33, tile=(8, 2, 4)), [0, 1], 1, 0),
]


def run_structured(g: DeviceRun, mask, rt, rs):
    a, d, wl = g.att, g.desc, g.wl
    rows = wl.batch * wl.heads * wl.n_video_tiles
    row_ptr = torch.full((rows + 1,), -7, dtype=torch.int64, device="cuda")
    col = torch.full((bsa.structured_entries(d, mask, rt, rs),), -7, dtype=torch.int32, device="cuda")
    bsa.plan_structured(d, mask, rt, rs, row_ptr, col)
    o = torch.empty_like(a.q_t)
    lse = torch.empty_like(a.lse)
    bsa.forward_csr(d, a.q_t, a.k_f, a.v_f, row_ptr, col, o, lse, workspace=a.workspace)
    torch.cuda.synchronize()
    return row_ptr.cpu().numpy(), col.cpu().numpy(), o, lse


def tile_grid(wl):
    return tuple(g // t for g, t in zip(wl.grid, wl.tile))


def check_slices(wl, g, q, k, v, row_ptr, col, o, lse, slices, n_tiles=None, seed=0):
    npf, scale = wl.n_prefix, float(np.float32(wl.scale))
    perm = g.perm()
    n = wl.n_video_tiles
    nqt = wl.n_tokens // 64
    rng = np.random.default_rng(seed)
    for b, h in slices:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        qt, kt, vt = (oracle.gather(sl(x), perm[b:b + 1], npf)[0, 0] for x in (q, k, v))
        r0 = (b * wl.heads + h) * n
        rp = row_ptr[r0:r0 + n + 1] - row_ptr[r0]
        cl = col[row_ptr[r0]:row_ptr[r0 + n]]
        tiles = (np.arange(nqt) if n_tiles is None else np.sort(rng.choice(nqt, n_tiles, replace=False))).astype(
            np.int32)
        ref, ref_lse = oracle.attention_csr(qt, kt, vt, npf, rp, cl, scale, tiles)
        ob = to_bits(o[b, h]).reshape(nqt, 64, wl.head_dim)[tiles]
        mx, mean = check_output(ob, ref, f"b{b} h{h}")
        check_lse(lse[b, h].cpu().numpy().reshape(nqt, 64)[tiles], ref_lse, qt.reshape(nqt, 64, -1)[tiles], kt, scale,
                  f"lse b{b} h{h}")
        print(f"[attention b{b} h{h}] rows {rp[-1] // n} tiles on average, max|err| {mx:.2e} mean {mean:.2e}",
              flush=True)


@pytest.mark.parametrize("wl,mask,rt,rs", CASES, ids=[c[0].name for c in CASES])
def test_structured_matches_oracle(wl, mask, rt, rs):
    print(f"\n[case] {wl} mask={mask} rt={rt} rs={rs}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    row_ptr, col, o, lse = run_structured(g, mask, rt, rs)
    ref_ptr, ref_col = oracle.plan_structured(tile_grid(wl), mask, rt, rs, wl.batch)
    assert np.array_equal(row_ptr, ref_ptr) and np.array_equal(col, ref_col)
    check_slices(wl, g, q, k, v, row_ptr, col, o, lse,
                 [(b, h) for b in range(wl.batch) for h in range(wl.heads)])


def test_structured_rejects_dynamic_tiles():
    d = bsa.make_desc(1, 2, 64, (8, 8, 8), 1, dynamic=True)
    rp = torch.zeros(17, dtype=torch.int64, device="cuda")
    cl = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(bsa.BsaError):
        bsa.plan_structured(d, [0, 1], 1, 1, rp, cl)


def test_prism720p_structured_sampled():
    """Full size: heads alternately spatial (radius 1 tile-frame) and temporal
    (radius 2 tiles); lists in full, attention on sampled slices."""
    wl = S.WORKLOADS["prism720p"]
    mask = [h % 2 for h in range(wl.heads)]
    print(f"\n[case] {wl} mask={mask} rt=1 rs=2", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    row_ptr, col, o, lse = run_structured(g, mask, 1, 2)
    ref_ptr, ref_col = oracle.plan_structured(tile_grid(wl), [0, 1], 1, 2, 1)
    n = wl.n_video_tiles
    sp_ptr, tm_ptr = ref_ptr[:n + 1], ref_ptr[n:] - ref_ptr[n]
    sp_col, tm_col = ref_col[:ref_ptr[n]], ref_col[ref_ptr[n]:]
    for b in range(wl.batch):
        for h in range(wl.heads):
            r0 = (b * wl.heads + h) * n
            rp = row_ptr[r0:r0 + n + 1] - row_ptr[r0]
            cl = col[row_ptr[r0]:row_ptr[r0 + n]]
            ep, ec = (sp_ptr, sp_col) if mask[h] == 0 else (tm_ptr, tm_col)
            assert np.array_equal(rp, ep) and np.array_equal(cl, ec), (b, h)
    check_slices(wl, g, q, k, v, row_ptr, col, o, lse, [(0, 0), (1, 1), (1, 6)], n_tiles=12, seed=5)
    del g, o, lse
    torch.cuda.empty_cache()
