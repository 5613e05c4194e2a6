"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant edits one line of the oracle's source text (a plausible slip: a
flipped tie rule, an unstable sort, float32 instead of exact arithmetic, a
transposed index ...), loads the edited copy as a separate module, and runs
every pin on it.  The real oracle is not touched.
"""
import inspect
import types

import pytest

import oracle_pins as pins
from oracle import eplb_oracle

MUTANTS = {
    "policy_condition_flipped": ("if num_groups % num_nodes == 0:", "if num_nodes % num_groups == 0:"),
    "sort_ties_descending_index": ("order = sorted(range(n), key=lambda i: weights[i], reverse=True)",
                                   "order = sorted(range(n), key=lambda i: (weights[i], i), reverse=True)"),
    "lightest_first": ("order = sorted(range(n), key=lambda i: weights[i], reverse=True)",
                       "order = sorted(range(n), key=lambda i: weights[i])"),
    "pack_tie_to_highest": ("key=lambda p: (pack_sum[p], p))", "key=lambda p: (pack_sum[p], -p))"),
    "pack_heaviest_open": ("target = min(open_packs", "target = max(open_packs"),
    "no_identity_when_one_per_pack": ("if per_pack == 1:", "if per_pack == 0:"),
    "replicate_tie_to_highest": ("if val > best_val:", "if val >= best_val:"),
    "replicate_float32": ("val = Fraction(loads[i], count[i])",
                          "val = np.float32(loads[i]) / np.float32(count[i])"),
    "replica_rank_after_increment": ("rank.append(count[best])", "rank.append(count[best] - 1)"),
    "mlog_transposed": ("base = (node_of_group[g] * groups_per_node + slot_of_group[g]) * S",
                        "base = (slot_of_group[g] * Np + node_of_group[g]) * S"),
    "step3_without_division": ("per_replica = [Fraction(u[local_phy[j]], count[local_phy[j]]) for j in range(Pn)]",
                               "per_replica = [Fraction(u[local_phy[j]], 1) for j in range(Pn)]"),
    "step3_float32": ("per_replica = [Fraction(u[local_phy[j]], count[local_phy[j]]) for j in range(Pn)]",
                      "per_replica = [np.float32(u[local_phy[j]]) / np.float32(count[local_phy[j]]) for j in range(Pn)]"),
    "pid_transposed": ("pid = n * Pn + gpu_of[j] * ppr + pos_of[j]",
                       "pid = n * Pn + pos_of[j] * RKn + gpu_of[j]"),
    "overflow_uses_max_count": ("if lcm(*count) * sum(u) >= SUM_LIMIT:", "if max(count) * sum(u) >= SUM_LIMIT:"),
    "load_bound_exclusive": ("(x < 0 or x > LOAD_MAX)", "(x < 0 or x >= LOAD_MAX)"),
    "capacity_off_by_one": ("if X < 1 + (P - E) // Np:", "if X < (P - E) // Np:"),
    "hist_drops_expert_zero": ("ok = (flat >= 0) & (flat < E)", "ok = (flat > 0) & (flat < E)"),
    "window_oldest_steps": ("recent = step_hists[-W:]", "recent = step_hists[:W]"),
    "redirect_by_k": ("t = np.arange(T, dtype=np.int64)[:, None]", "t = np.arange(K, dtype=np.int64)[None, :]"),
    "ema_rounds_up": ("out = [e - (e >> shift) + c for e, c in zip(ema, cnt)]",
                      "out = [e - (-(-e >> shift)) + c for e, c in zip(ema, cnt)]"),
    "rearrange_freed_descending": ("freed = [s for s in slots if s not in used_old]",
                                   "freed = [s for s in reversed(slots) if s not in used_old]"),
    "rearrange_keeps_one_less": ("for q, p in zip(old_e, new_e):", "for q, p in zip(old_e[1:], new_e[1:]):"),
    "rearrange_node_before_rank": ("if same_rank:\n                src[s], cls = same_rank[0], 0",
                                   "if same_rank and not same_node:\n                src[s], cls = same_rank[0], 0"),
    "rearrange_highest_source": ("src[s], cls = holders[0], 2", "src[s], cls = holders[-1], 2"),
    "rearrange_node_of_rank": ("same_node = [q for q in holders if q // per_node == s // per_node]",
                               "same_node = [q for q in holders if q // ppr // N == s // ppr // N]"),
    "lp_capacity_is_one": ("cap[home[x]][g] += cnt[x]", "cap[home[x]][g] += 1"),
    "lp_edge_reversed": ("cap[home[x]][g] += cnt[x]", "cap[g][home[x]] += cnt[x]"),
    "lp_search_upper_off": ("lo, hi = 0, max(base)", "lo, hi = 0, max(base) - 1"),
    "lp_split_ignores_count": ("f = min(net, c[x])", "f = net"),
    "lp_sink_room_too_big": ("r[v][t] = max(0, lam - base[v])", "r[v][t] = max(0, lam - base[v] + 1)"),
    "lp_redirect_keeps_first": ("to_rep = valid & (slot[e] >= 0) & (occ < fx[e])",
                                "to_rep = valid & (slot[e] >= 0) & (occ >= fx[e])"),
    "rank_load_ignores_count": ("r = [sum((Fraction(w[phy[g * ppr + s]], c[phy[g * ppr + s]])",
                                "r = [sum((Fraction(w[phy[g * ppr + s]], 1)"),
}


def _mutant_module(old, new):
    src = inspect.getsource(eplb_oracle)
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant_module(*MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:                      # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
