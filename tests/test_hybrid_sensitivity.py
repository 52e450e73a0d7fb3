"""CPU: the chunk-hybrid parity checks can see a mistake in either partial.

The GPU tests compare the merged output (and LSE) of a chunk-hybrid call with
the oracle.  Whether that comparison would notice a kernel that gets one of
the two partials wrong depends on how much weight each partial carries, which
depends on the softmax scale (MobileWan review, Sec. 3.2: the softmax term
e^{s} and the linear term phi(q)^T z are normalised jointly).  Here mistakes
are planted in the oracle's own partials at the shapes and scales of
tests/test_gpu_hybrid.py (12090 tokens on the 31 x 15 x 26 grid, chunks of
1170, or of 1560 with 780 tokens of overlap; two heads instead of 24, same
per-head statistics), and each mutated output must fail the parity bar that
those GPU tests apply.  Only oracle/ and the seeded generators are used.

Mutations: the softmax numerator dropped in chunks >= 1; the softmax taken
over the previous chunk's keys; the linear numerator dropped; the linear
state including the query's own chunk; the state one chunk behind; phi taken
of the softmax-scaled query (scale * log2 e * q).
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as WL

BF16_MAX, BF16_MEAN, BF16_REL, LSE_BF16 = 2e-2, 2e-3, 1e-2, 1e-2  # tests/parity.py


def _fails_bar(o, lse, o_ref, lse_ref, C):
    """The GPU tests' bar: absolute and relative errors over all rows, the
    relative error of every chunk on its own, and the LSE."""
    e = np.abs(o - o_ref)
    rel = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
    rel_c = max(np.linalg.norm(o[:, c0:c0 + C] - o_ref[:, c0:c0 + C]) / np.linalg.norm(o_ref[:, c0:c0 + C])
                for c0 in range(0, o.shape[1], C))
    both = np.isneginf(lse) & np.isneginf(lse_ref)
    dl = np.abs(np.where(both, 0.0, lse - lse_ref))
    return bool(e.max() > BF16_MAX or e.mean() > BF16_MEAN or rel > BF16_REL or rel_c > BF16_REL
                or dl.max() > LSE_BF16), \
        f"max {e.max():.2e} mean {e.mean():.2e} relF {rel:.2e} worst chunk relF {rel_c:.2e} lse {dl.max():.2e}"


@pytest.fixture(scope="module", params=[5, 8])
def case(request):
    w = WL.WORKLOADS[request.param]
    rng = np.random.default_rng(w.seed)
    shape = (1, w.tokens, 2, w.head_dim)
    q, k, v = (WL.draw(shape, rng, "bf16") for _ in range(3))
    wq, wk = O.rope_qk(q.values, k.values, w.grid, w.pairs)
    return w, wq, wk, v.values


def _linear(q, k, v, c0, c1, upto, qscale=1.0):
    """Linear partial (o_l, lse_l) of queries [c0, c1) over keys [0, upto)."""
    fq = O.phi(q[:, c0:c1] * qscale)
    fk = O.phi(k[:, :max(upto, 0)])
    S = np.matmul(fk.transpose(0, 2, 3, 1), v[:, :max(upto, 0)].transpose(0, 2, 1, 3))  # [B, H, D, D]
    z = fk.sum(axis=1)                                                                     # [B, H, D]
    num = np.matmul(fq.transpose(0, 2, 1, 3), S).transpose(0, 2, 1, 3)                  # [B, n, H, D]
    den = np.einsum("bnhd,bhd->bhn", fq, z)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(den.transpose(0, 2, 1)[..., None] > 0, num / den.transpose(0, 2, 1)[..., None], 0.0)
        l = np.where(den > 0, np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return o, l


def _mutations(w, wq, wk, v, scale):
    C, Ov, L = w.chunk_tokens, w.overlap_tokens, w.tokens
    o_s, l_s, o_l, l_l = O.hybrid_partials(wq, wk, v, C, scale=scale, overlap=Ov)
    ref = O.lse_merge(o_s, l_s, o_l, l_l)
    chunks = [(c0, min(L, c0 + C)) for c0 in range(C, L, C)]   # chunks >= 1
    out = {}
    m = o_s.copy()
    m[:, C:] = 0.0
    out["softmax numerator dropped"] = O.lse_merge(m, l_s, o_l, l_l)
    m, ml = o_s.copy(), l_s.copy()
    for c0, c1 in chunks:
        a, b = max(0, c0 - C - Ov), c0
        oc, lc = O.attention(wq[:, c0:c1], wk[:, a:b], v[:, a:b], scale)
        m[:, c0:c1], ml[:, :, c0:c1] = oc, lc
    out["softmax over the previous chunk"] = O.lse_merge(m, ml, o_l, l_l)
    out["linear numerator dropped"] = O.lse_merge(o_s, l_s, np.zeros_like(o_l), l_l)
    for name, upto, qs in (("state includes the own chunk", lambda c0, c1: c1, 1.0),
                           ("state one chunk behind", lambda c0, c1: c0 - Ov - C, 1.0),
                           ("phi of the scaled query", lambda c0, c1: c0 - Ov, scale * math.log2(math.e))):
        m, ml = o_l.copy(), l_l.copy()
        for c0, c1 in chunks:
            oc, lc = _linear(wq, wk, v, c0, c1, upto(c0, c1), qs)
            m[:, c0:c1], ml[:, :, c0:c1] = oc, lc
        out[name] = O.lse_merge(o_s, l_s, m, ml)
    return ref, out


# (workload, scale) -> mutations the bar must catch there.  At the default
# 1/sqrt(D) the linear partial holds ~99% of the weight after chunk 0: over
# all rows a dropped softmax numerator stays under the relative guard at
# workload 5 (8.1e-3), and only the per-chunk guard sees it (1.6e-2 in the
# worst chunk); at the larger, balanced scales every guard does.
LINEAR = ["linear numerator dropped", "state includes the own chunk", "state one chunk behind",
          "phi of the scaled query"]
SOFTMAX = ["softmax numerator dropped", "softmax over the previous chunk"]
EXPECT = {(5, "default"): SOFTMAX + LINEAR, (5, 0.35): SOFTMAX + LINEAR, (8, "default"): SOFTMAX + LINEAR,
          (8, 0.32): SOFTMAX + LINEAR}


@pytest.mark.parametrize("scale", ["default", "balanced"])
def test_planted_mistakes_fail_the_bar(case, scale):
    w, wq, wk, v = case
    key = (w.number, "default") if scale == "default" else next(k for k in EXPECT if k[0] == w.number and k[1] != "default")
    sc = 1.0 / math.sqrt(w.head_dim) if scale == "default" else key[1]
    ref, muts = _mutations(w, wq, wk, v, sc)
    report = []
    for name, (o, lse) in muts.items():
        caught, stats = _fails_bar(o, lse, *ref, w.chunk_tokens)
        report.append(f"{name}: {'caught' if caught else 'missed'} ({stats})")
        if name in EXPECT[key]:
            assert caught, f"workload {w.number}, scale {sc:.4f}: '{name}' passes the bar ({stats})"
    print(f"\nworkload {w.number} scale {sc:.4f}:\n  " + "\n  ".join(report))
