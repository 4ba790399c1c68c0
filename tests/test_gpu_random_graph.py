"""Graph replay over seeded random batch sequences: for each case, one
PKA_GRAPH_STABLE plan is captured into a HIP graph and replayed over four
batches of random sizes and lengths (one kind per plan: prefill or decode),
each replay bit-identical to an eager run and within tolerance of the
oracle (the checks of test_gpu_graph.py, on random shapes)."""
import pytest
import torch

from inputs import workloads as W
from tests.test_gpu_graph import _replay_batches

pytestmark = pytest.mark.gpu


def _batches(seed):
    g = torch.Generator().manual_seed(3000 + seed)
    pick = lambda xs: xs[int(torch.randint(0, len(xs), (1,), generator=g))]
    D, Hkv, G, ps = pick([64, 128]), pick([1, 2, 4]), pick([1, 2, 4, 6]), pick([1, 3, 4, 16])
    causal = bool(torch.rand(1, generator=g) < 0.75)
    decode = seed % 2 == 1
    num_pages = 9600 // ps + 80  # enough for 8 requests of up to 1199 keys
    ws = []
    for i in range(4):
        B = int(torch.randint(1, 9, (1,), generator=g))
        kv = [int(torch.randint(0, 1200, (1,), generator=g)) for _ in range(B)]
        qo = [1] * B if decode else [int(torch.randint(0, 200, (1,), generator=g)) for _ in range(B)]
        if not decode and max(qo) < 2:
            qo[0] = 2
        ws.append(W.build(f"rgraph{seed}_{i}", 3100 + 10 * seed + i, qo, kv, Hkv * G, Hkv, D, ps,
                          causal=causal, num_pages=num_pages))
    return ws


@pytest.mark.parametrize("seed", range(8))
def test_random_graph_replay(seed):
    ws = _batches(seed)
    w = ws[0]
    print(f"case {seed}: D={w.head_dim} Hq={w.num_qo_heads} Hkv={w.num_kv_heads} ps={w.page_size} "
          f"causal={w.causal} batches={[w.batch for w in ws]}", flush=True)
    _replay_batches(ws)
