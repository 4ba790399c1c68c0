"""GPU parity over seeded random batch shapes: group sizes, head dims, page
sizes, causal or not, split-KV on or off, bf16 or fp32 output, request
lengths from empty to a few hundred (query rows past the keys included),
paged and ragged K/V, and mixed prefill/decode batches in one launch or two.  Each case is small enough for the oracle and checked
on every row.  The cases are drawn from fixed seeds, so a failure names its
case and reproduces."""
import pytest
import torch

import paged_kv_cache_plan_amd as pka
from inputs import workloads as W
from tests.gpu_common import compare, oracle_paged, run_paged, run_ragged

pytestmark = pytest.mark.gpu

N_CASES = 160


def _case(seed):
    g = torch.Generator().manual_seed(1000 + seed)
    pick = lambda xs: xs[int(torch.randint(0, len(xs), (1,), generator=g))]
    D = pick([64, 128])
    Hkv = pick([1, 2, 4, 8])
    G = pick([1, 2, 3, 4, 5, 6, 8])
    ps = pick([1, 2, 3, 4, 5, 8, 16, 32, 64])
    causal = bool(torch.rand(1, generator=g) < 0.7)
    decode = bool(torch.rand(1, generator=g) < 0.3)
    B = int(torch.randint(1, 7, (1,), generator=g))
    kv, qo = [], []
    for _ in range(B):
        k = pick([0, 1, 2, 63, 64, 65]) if torch.rand(1, generator=g) < 0.3 else int(torch.randint(1, 700, (1,), generator=g))
        if decode:
            q = 1
        else:
            q = pick([0, 1]) if torch.rand(1, generator=g) < 0.2 else int(torch.randint(1, 300, (1,), generator=g))
        kv.append(k)
        qo.append(q)
    split = bool(torch.rand(1, generator=g) < 0.5)
    fp32 = bool(torch.rand(1, generator=g) < 0.3)
    ragged = bool(torch.rand(1, generator=g) < 0.25)
    # a mixed batch (prefill and single-token requests, one launch or two)
    mixed = (not decode and not ragged and B > 1) and pick([None, None, None, "one", "two"])
    if mixed:
        for i in range(0, B, 2):
            qo[i] = 1
    return dict(D=D, Hkv=Hkv, G=G, ps=ps, causal=causal, qo=qo, kv=kv, split=split, fp32=fp32, ragged=ragged,
                mixed=mixed or None)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    c = _case(seed)
    print(f"case {seed}: {c}", flush=True)
    w = W.build(f"rand{seed}", 2000 + seed, c["qo"], c["kv"], c["Hkv"] * c["G"], c["Hkv"], c["D"],
                1 if c["ragged"] else c["ps"], causal=c["causal"], ragged=c["ragged"], pool_slack=0.1)
    kw = dict(disable_split_kv=not c["split"], out_fp32=c["fp32"])
    if c["mixed"]:
        kw.update(mixed=True, mixed_two_launches=c["mixed"] == "two")
    if c["ragged"]:
        o, lse, info = run_ragged(w, **kw)
    else:
        o, lse, info = run_paged(w, **kw)
    kinds = (pka.PKA_KERNEL_PREFILL, pka.PKA_KERNEL_DECODE) + ((pka.PKA_KERNEL_MIXED,) if c["mixed"] else ())
    assert info["kernel"] in kinds
    compare(o, lse, *oracle_paged(w), f"case {seed}")
