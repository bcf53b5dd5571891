"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
some pin in test_oracle.py catches each one."""

import os
import types

import pytest

import test_oracle as T

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "fva_oracle.py")

MUTANTS = [
    ("tile inner order column-major",
     "tok = (ts[:, None, None] * H + ys[None, :, None]) * W + xs[None, None, :]",
     "tok = np.transpose((ts[:, None, None] * H + ys[None, :, None]) * W + xs[None, None, :], (0, 2, 1))",
     ["test_block_order_golden"]),
    ("unreorder ignores the permutation",
     "x[:, order, :, :] = np.transpose(y[:, :, :N, :], (0, 2, 1, 3))",
     "x[:, :, :, :] = np.transpose(y[:, :, :N, :], (0, 2, 1, 3))",
     ["test_reorder_roundtrip_and_padding"]),
    ("pool divides by the block size",
     "sum(axis=2) / (hi - lo)", "sum(axis=2) / BLK",
     ["test_pool_partial_last_block_uses_real_tokens_only"]),
    ("scores transposed",
     "np.matmul(qbar, np.swapaxes(kbar, -1, -2)) * scale",
     "np.matmul(kbar, np.swapaxes(qbar, -1, -2)) * scale",
     ["test_scores_rank_one_closed_form"]),
    ("scores miss the scale",
     "np.matmul(qbar, np.swapaxes(kbar, -1, -2)) * scale",
     "np.matmul(qbar, np.swapaxes(kbar, -1, -2))",
     ["test_scores_rank_one_closed_form"]),
    ("cut uses > instead of >=", "nstar = int(np.argmax(C >= target)) + 1",
     "nstar = int(np.argmax(C > target)) + 1", ["test_route_worked_examples"]),
    ("ties broken by descending index",
     "j = np.broadcast_to(np.arange(nB), flat.shape)",
     "j = np.broadcast_to(np.arange(nB)[::-1], flat.shape)",
     ["test_route_worked_examples"]),
    ("floor intersected instead of unioned",
     "n = min(nB, max(nstar, int(topk)))", "n = min(nB, min(nstar, int(topk)))",
     ["test_route_worked_examples", "test_route_bruteforce_minimal_prefix"]),
    ("cumulative sum in index order, not importance order",
     "e = np.exp(s - s[0])", "e = np.exp(rows[r].astype(np.float64) - s[0])",
     ["test_route_worked_examples"]),
    ("top-up ties j before i", "pick = np.lexsort((fj, fi, -s))[:need]",
     "pick = np.lexsort((fi, fj, -s))[:need]", ["test_sasa_topup_bruteforce"]),
    ("top-up takes the lowest scores", "pick = np.lexsort((fj, fi, -s))[:need]",
     "pick = np.lexsort((fj, fi, s))[:need]", ["test_sasa_topup_bruteforce"]),
    ("attention keeps padded keys",
     "keys = np.concatenate([np.arange(j * BLK, min((j + 1) * BLK, N)) for j in sel])",
     "keys = np.concatenate([np.arange(j * BLK, (j + 1) * BLK) for j in sel])",
     ["test_zero_queries_average_selected_real_values"]),
    ("attention drops the scale", "logits = (q @ k.T) * scale", "logits = (q @ k.T)",
     ["test_sparse_output_equals_dense_on_selected_keys_only"]),
    ("queue lightest-first", "key=lambda t: (-int(flat[t]), t)",
     "key=lambda t: (int(flat[t]), t)", ["test_heaviest_first_order"]),
    ("Hilbert without Gray encoding", "    for i in range(1, 3):\n        x[i] ^= x[i - 1]\n",
     "", [("test_hilbert_curve_is_a_face_adjacent_walk_of_the_cube", {"bits": 3})]),
    ("Hilbert exchange replaced by inversion",
     "                swap = (x[0] ^ x[i]) & low\n                x[0] ^= swap\n                x[i] ^= swap",
     "                x[0] ^= low",
     [("test_hilbert_curve_is_a_face_adjacent_walk_of_the_cube", {"bits": 3})]),
    ("Hilbert tiles in raster order", "    return sorted(ids, key=lambda i: key[i])",
     "    return ids", ["test_hilbert_tile_order_restricts_the_cube_walk"]),
    ("lse keeps padded keys",
     "    return np.concatenate([np.arange(j * BLK, min((j + 1) * BLK, N)) for j in sel])",
     "    return np.concatenate([np.arange(j * BLK, (j + 1) * BLK) for j in sel])",
     ["test_lse_full_mask_equals_library_logsumexp"]),
    ("lse forgets to add the max back",
     "return m + np.log(np.exp(logits - m[:, None]).sum(axis=1))",
     "return np.log(np.exp(logits - m[:, None]).sum(axis=1))",
     ["test_lse_full_mask_equals_library_logsumexp"]),
    ("lse reads the first query rows",
     "logits = (qr[lo:hi].astype(np.float64) @ kr[keys]",
     "logits = (qr[:hi - lo].astype(np.float64) @ kr[keys]",
     ["test_lse_full_mask_equals_library_logsumexp"]),
    ("lse drops the scale", "@ kr[keys].astype(np.float64).T) * scale",
     "@ kr[keys].astype(np.float64).T)", ["test_lse_full_mask_equals_library_logsumexp"]),
    ("recall inverted",
     "np.exp(np.asarray(lse_selected, np.float64) - np.asarray(lse_all, np.float64))",
     "np.exp(np.asarray(lse_all, np.float64) - np.asarray(lse_selected, np.float64))",
     ["test_recall_equals_dense_mass_on_selected_blocks"]),
    ("margin not normalized by Z", "margin[r] = m / Z", "margin[r] = m",
     ["test_route_margin_worked_examples"]),
    ("margin ignores the n*-1 side", "m = min(m, abs(C[nstar - 2] - target))", "m = m",
     ["test_route_margin_worked_examples"]),
    ("head workload always zero",
     "mask.reshape(mask.shape[0], mask.shape[1], -1).sum(axis=-1).astype(np.int64)",
     "mask.reshape(mask.shape[0], mask.shape[1], -1).sum(axis=-1).astype(np.int64) * 0",
     ["test_head_workload_hand_worked"]),
    ("head workload counts rows, not pairs",
     "mask.reshape(mask.shape[0], mask.shape[1], -1).sum(axis=-1).astype(np.int64)",
     "mask.any(axis=-1).sum(axis=-1).astype(np.int64)",
     ["test_head_workload_hand_worked"]),
    ("sasa budget cap ignored",
     "out[h] = min(max(want, int(W[h])), max(head_cap, int(W[h])))",
     "out[h] = max(want, int(W[h]))",
     ["test_sasa_budget_cap_hand_worked", "test_sasa_budget_invariants_when_the_cap_binds"]),
    ("sasa budget cap lowers a head below its workload",
     "out[h] = min(max(want, int(W[h])), max(head_cap, int(W[h])))",
     "out[h] = min(want, head_cap)",
     ["test_sasa_budget_cap_hand_worked", "test_sasa_budget_invariants_when_the_cap_binds"]),
    ("sasa remainder to the highest head ids", "want = int(W[h]) + q + (1 if k < rem else 0)",
     "want = int(W[h]) + q + (1 if k >= len(hs) - rem else 0)",
     ["test_sasa_budget_cap_hand_worked"]),
    ("CU named without shader-engine bits", "((r[2] >> 8) & 0xFF)", "((r[2] >> 8) & 0xF)",
     ["test_imbalance_hand_worked_trace"]),
    ("CU named with wave and SIMD bits", "((r[2] >> 8) & 0xFF)", "(r[2] & 0xFFFF)",
     ["test_imbalance_hand_worked_trace"]),
    ("XCC_ID not masked", "unit = ((r[1] & 0xF) << 8)", "unit = ((r[1]) << 8)",
     ["test_imbalance_hand_worked_trace"]),
    ("CU mean over the units seen only",
     "loads = list(busy.values()) + [0] * (n_units - len(busy))", "loads = list(busy.values())",
     ["test_imbalance_hand_worked_trace"]),
    ("imbalance as max over min", "return max(L) / mean", "return max(L) / min(L)",
     ["test_load_imbalance_rank_form"]),
    ("slot imbalance without the slot count", "return span * slots / total",
     "return span / total", ["test_imbalance_hand_worked_trace"]),
]


def _mutant_module(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("fva_oracle_mutant")
    mod.__dict__["__file__"] = SRC
    exec(compile(src.replace(old, new, 1), SRC + "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutant(name, old, new, catchers, monkeypatch):
    monkeypatch.setattr(T, "O", _mutant_module(old, new))
    # every catcher passes on the real oracle (so a catch is the mutant's doing)
    caught = []
    for c in catchers:
        t, kw = (c, {}) if isinstance(c, str) else c
        try:
            getattr(T, t)(**kw)
        except AssertionError:
            caught.append(t)
    assert caught, f"no pin caught mutant: {name}"
