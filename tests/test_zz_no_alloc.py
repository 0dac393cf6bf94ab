"""kvsel_gather_attn_noalloc (the allocation-free gathered attention, whose
split records live in the library's fixed per-device array) gives the same
attention as kvsel_gather_attn on two calls in a row, the second smaller
than the first, so a record left over from the first call cannot be read by
the second.  Both calls split their (sequence, kv head) pairs over several
work-groups, so the fixed array is used."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.gpu_util import assert_attn, log_case, need_gpu, random_paged

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / math.sqrt(128)


def _case(seed, batch, hkv, G, lens, seg, k):
    from decode_focal_layer_amd import kvsel
    rng = np.random.default_rng(seed)
    max_len = max(lens)
    kp, vp, table = random_paged(rng, batch, hkv, max_len, DEV)
    kv = kvsel.KV(kp, vp, torch.from_numpy(table).to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                  torch.zeros(batch, dtype=torch.int32, device=DEV), torch.full((batch,), seg, dtype=torch.int32, device=DEV),
                  max_seq_len=max_len, max_seg_len=seg, min_seg_len=seg)
    hq = hkv * G
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16).to(DEV)
    keys = torch.rand((batch * hkv, seg), generator=torch.Generator().manual_seed(seed + 1))
    idx = keys.argsort(dim=1)[:, :k].sort(dim=1).values.to(torch.int32).view(batch, hkv, k).to(DEV)
    return kv, q, idx, hq, table


@pytest.mark.parametrize("order", ["large_then_small"])
def test_gather_attn_noalloc_matches_gather_attn(order):
    need_gpu()
    from decode_focal_layer_amd import kvsel
    cases = [dict(seed=501, batch=3, hkv=4, G=2, lens=[3000, 2500, 2900], seg=2000, k=100),
             dict(seed=502, batch=1, hkv=2, G=4, lens=[1700], seg=1200, k=40)]
    for c in cases:
        kv, q, idx, hq, table = _case(**c)
        ws_need = kvsel.attn_workspace(kv, hq, c["k"])
        assert ws_need > 65536, "the case must split its pairs (records in the scratch)"
        ref_o = torch.zeros((c["batch"], hq, 128), dtype=torch.float32, device=DEV)
        ref_l = torch.zeros((c["batch"], hq), dtype=torch.float32, device=DEV)
        out = torch.full((c["batch"], hq, 128), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((c["batch"], hq), float("nan"), dtype=torch.float32, device=DEV)
        log_case("noalloc", c["seed"], c["batch"], c["hkv"], c["G"], c["lens"], c["k"])
        kvsel.gather_attn(kv, q, hq, SCALE, idx, c["k"], ref_o, ref_l)
        kvsel.gather_attn_noalloc(kv, q, hq, SCALE, idx, c["k"], out, lse)
        torch.cuda.synchronize()
        assert_attn(out.cpu().numpy(), ref_o.cpu().numpy(), f"noalloc vs gather_attn seed {c['seed']}")
        assert (lse - ref_l).abs().max().item() < 1e-4
        # and against the oracle on one (sequence, kv head)
        kc, vc = kv.k_pool.cpu(), kv.v_pool.cpu()
        G = c["G"]
        b, g = c["batch"] - 1, c["hkv"] - 1
        n = c["lens"][b]
        Kl, Vl = O.logical_rows(kc, table[b], g, n), O.logical_rows(vc, table[b], g, n)
        ref, _ = O.attention(O.widen(q[b, g * G:(g + 1) * G].cpu()), Kl, Vl,
                             O.kept_rows(idx[b, g].cpu().numpy(), 0, c["seg"], n), SCALE)
        assert_attn(out[b, g * G:(g + 1) * G].cpu().numpy(), ref, f"noalloc vs oracle seed {c['seed']}")
