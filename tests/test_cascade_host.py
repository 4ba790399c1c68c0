"""The cascade's host-side size query (pka_cascade_workspace_size): level
layouts that are accepted, the sizes they report, and the errors it gives for
malformed levels.  Pure host code: no GPU."""
import pytest
import torch

import paged_kv_cache_plan_amd as pka

Hq, Hkv, D, PS = 8, 2, 128, 16


def _level(qo, kv_tokens, first_page=0):
    """One level: contiguous query groups with the given row counts, group g
    over kv_tokens[g] keys in fresh pages."""
    qo_indptr, kv_indptr, idx, last = [0], [0], [], []
    page = first_page
    for nq, nk in zip(qo, kv_tokens):
        qo_indptr.append(qo_indptr[-1] + nq)
        n = (nk + PS - 1) // PS
        idx += list(range(page, page + n))
        page += n
        kv_indptr.append(len(idx))
        last.append(0 if nk == 0 else nk - (n - 1) * PS)
    t = lambda x: torch.tensor(x, dtype=torch.int32)
    return (t(qo_indptr), t(kv_indptr), t(idx), t(last)), page


def _two_levels(qo_lens=(5, 1, 9), prefix=300, own=(40, 17, 9)):
    l0, p = _level([sum(qo_lens)], [prefix])
    l1, _ = _level(list(qo_lens), list(own), p)
    return [l0, l1]


def test_sizes_cover_every_level_and_the_states():
    levels = _two_levels()
    a, b = pka.cascade_workspace_size(levels, Hq, Hkv, D, PS)
    total_q = 15
    parts = [pka.workspace_size(l[0], l[1], l[3], Hq, Hkv, D, PS, causal=(i == 1), flags=pka.PKA_OUT_FP32)
             for i, l in enumerate(levels)]
    assert a >= sum(x for x, _ in parts)
    # every level's float workspace plus fp32 states (v and s) of each level
    assert b >= sum(y for _, y in parts) + 2 * total_q * Hq * (D + 1) * 4


def test_states_grow_with_levels():
    two = pka.cascade_workspace_size(_two_levels(), Hq, Hkv, D, PS)[1]
    l0, p = _level([15], [300])
    l1, p = _level([8, 7], [60, 70], p)
    l2, _ = _level([5, 1, 9], [40, 17, 9], p)
    three = pka.cascade_workspace_size([l0, l1, l2], Hq, Hkv, D, PS)[1]
    assert three > two + 15 * Hq * D * 4


def test_one_level_is_a_plain_plan():
    (l0, _) = _level([5, 1, 9], [40, 17, 9])
    a, b = pka.cascade_workspace_size([l0], Hq, Hkv, D, PS)
    assert a > 0 and b > 0


@pytest.mark.parametrize("case", ["total_q", "flags", "no_levels", "too_many", "nnz", "causal_short", "heads"])
def test_size_query_errors(case):
    levels = _two_levels()
    kw = {}
    if case == "total_q":  # level 1 covers fewer query rows than level 0
        levels[1], _ = _level([5, 1, 8], [40, 17, 9], 100)
    elif case == "flags":  # only PKA_OUT_FP32 / PKA_DISABLE_SPLIT_KV are cascade flags
        L = pka.load_library()
        lv = pka._level_arrays(levels)
        import ctypes
        a, b = ctypes.c_size_t(), ctypes.c_size_t()
        code = L.pka_cascade_workspace_size(2, lv.qo, lv.kvp, lv.last, lv.batch, Hq, Hkv, D, PS, 1,
                                            pka.PKA_GRAPH_STABLE, ctypes.byref(a), ctypes.byref(b))
        assert code == pka.PKA_ERR_INVALID_ARG
        assert "PKA_OUT_FP32" in L.pka_last_error().decode()
        return
    elif case == "no_levels":
        L = pka.load_library()
        import ctypes
        a, b = ctypes.c_size_t(), ctypes.c_size_t()
        code = L.pka_cascade_workspace_size(0, None, None, None, None, Hq, Hkv, D, PS, 1, 0, ctypes.byref(a),
                                            ctypes.byref(b))
        assert code == pka.PKA_ERR_INVALID_ARG
        return
    elif case == "too_many":
        levels = [levels[0]] * 65
    elif case == "nnz":  # kv_indptr[batch] disagrees with kv_indices' length
        qo, kvp, idx, last = levels[1]
        levels[1] = (qo, kvp, idx[:-1], last)
        L = pka.load_library()
        lv = pka._level_arrays(levels)
        import ctypes
        null = ctypes.c_void_p()
        code = L.pka_cascade_create(2, lv.qo, lv.kvp, lv.kvi, lv.last, lv.batch, lv.nnz, 1000, Hq, Hkv, D, PS, 1,
                                    0.0, 0, ctypes.c_void_p(1), 1 << 30, ctypes.c_void_p(1), 1 << 30, None,
                                    ctypes.byref(null))
        assert code == pka.PKA_ERR_INVALID_ARG and not null.value
        assert "nnz_pages" in L.pka_last_error().decode()
        return
    elif case == "causal_short":  # the last level must hold each request's own query tokens
        levels[1], _ = _level([5, 1, 9], [4, 17, 9], 100)
    elif case == "heads":
        kw = {"num_kv_heads": 3}
    with pytest.raises(pka.PkaError):
        pka.cascade_workspace_size(levels, Hq, kw.get("num_kv_heads", Hkv), D, PS, causal=True)


def test_non_causal_accepts_short_last_level():
    levels = _two_levels()
    levels[1], _ = _level([5, 1, 9], [4, 17, 9], 100)
    a, b = pka.cascade_workspace_size(levels, Hq, Hkv, D, PS, causal=False)
    assert a > 0 and b > 0
