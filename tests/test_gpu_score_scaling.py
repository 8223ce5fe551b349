"""The tile scores are bilinear in the two MLP branches, and the kernels keep that exactly.

y = GELU(desc W1) W2 is linear in W2, and a score is scale * y_q . y_k; so with the Q
branch's W2 times 2 every score doubles, and with the K branch's W2 times 4 every score
quadruples, bit for bit (a power-of-two factor is exact in every fp32 product and sum while
nothing overflows), and the kept lists do not move (the order of the scores is kept
exactly, ties included).  The pipeline's own weights alias the two branches; here they are
separate tensors, so a kernel that read one branch's weights for the other fails.  Every
row of every head, at full size (the scores of all query tiles are written)."""
import numpy as np
import pytest
import torch

from workloads import get, make

pytestmark = pytest.mark.gpu

V = pytest.importorskip("video_dit_block_head_amd")
from video_dit_block_head_amd.pipeline import SparseAttention  # noqa: E402


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", ["small", "large", "long"])
def test_scores_bilinear_in_the_branches(name):
    cfg = get(name)
    say(f"[gpu-score-scaling] {name}: generating")
    wl = make(cfg)
    geom = V.Geom(cfg.batch, cfg.heads, cfg.head_dim, cfg.grid, cfg.tile, wl.shapes)
    up = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    q, k = up(wl.q), up(wl.k)
    w1, w2 = torch.from_numpy(wl.w1), torch.from_numpy(wl.w2)
    kk = cfg.topk[0]
    B, H, nt = cfg.batch, cfg.heads, cfg.n_tiles
    runs = {}
    for tag, fq, fk in (("base", 1.0, 1.0), ("q2", 2.0, 1.0), ("k4", 1.0, 4.0)):
        sa = SparseAttention(geom, torch.bfloat16, w1, w2 * fq, w1_k=w1.clone(), w2_k=w2 * fk,
                             score_scale=cfg.score_scale)
        sa.gather(q, k, q)  # V unused here
        scores = torch.empty((B, H, nt, nt), dtype=torch.float32, device="cuda")
        idx = sa.score(kk, scores=scores)
        torch.cuda.synchronize()
        runs[tag] = (scores, idx.clone())
        del sa
    s0, i0 = runs["base"]
    for tag, f in (("q2", 2.0), ("k4", 4.0)):
        s, i = runs[tag]
        assert torch.equal(s, s0 * f), (name, tag)
        assert torch.equal(i, i0), (name, tag)
        say(f"[gpu-score-scaling] {name}: {tag}: every score times {f:g} bit for bit, lists identical")
