"""Plant plausible mistakes in copies of the oracle and require that a pin fails.

Each mutation is a textual edit of the oracle's source, executed as a separate
module on the CPU.  If every pin still passed on a mutant, the pins would not
be able to tell that mistake from the intended method.
"""
import inspect
import types

import pytest

import oracle.spin_oracle as om
from tests import oracle_pins as P

MUTATIONS = {
    "score_scale": ("/ math.sqrt(self.D))\n", "/ self.D)\n"),
    "group_map_strided": ("q[b, h * self.G:(h + 1) * self.G].sum(axis=0)", "q[b, h::self.Hkv].sum(axis=0)"),
    "group_sum_not_mean": ("].sum(axis=0) / self.G", "].sum(axis=0)"),
    "tie_break_high_index": ("np.lexsort((np.arange(len(s)), -s))", "np.lexsort((-np.arange(len(s)), -s))"),
    "bucket_reversed": ("return (NUM_BUCKETS - 1) - min(NUM_BUCKETS - 1, t - last_use)",
                        "return min(NUM_BUCKETS - 1, t - last_use)"),
    "bucket_no_saturation": ("return (NUM_BUCKETS - 1) - min(NUM_BUCKETS - 1, t - last_use)",
                             "return max(0, (NUM_BUCKETS - 1) - (t - last_use) // 2)"),
    "cutoff_bucket_high_slots_first": ("for c in cands:  # ascending slot order", "for c in reversed(cands):"),
    "mandatory_evictable": ("and c not in mandatory_slots]", "]"),
    "hit_not_refreshed": ("self.last_use[b, c] = t\n                    mand.add(c)", "mand.add(c)"),
    "evict_one_extra": ("need = max(0, n_resident + len(misses) - self.budget[b])",
                        "need = max(0, n_resident + len(misses) - self.budget[b] + 1)"),
    "budget_ignored": ("need = max(0, n_resident + len(misses) - self.budget[b])",
                       "need = max(0, n_resident + len(misses) - self.C)"),
    "segment_never_freed": ("self.seg_live[s] == 0:\n                    self.directory[b, h, e] = FREE\n                    self.free_stack.append(int(s))",
                            "self.seg_live[s] == -5:\n                    pass"),
    "live_not_counted": ("self.seg_live[s] += 1", "pass"),
    "free_slots_descending": ("free_slots = [c for c in range(self.C) if self.owner[b, c] == FREE]",
                              "free_slots = [c for c in range(self.C - 1, -1, -1) if self.owner[b, c] == FREE]"),
    "canonical_heads_reversed": ("        for h in range(self.Hkv):\n            for p in sel_b[h]:",
                                 "        for h in reversed(range(self.Hkv)):\n            for p in sel_b[h]:"),
    "summary_counts_padding": ("rows.append(K[: req.page_tokens(i, j)])", "rows.append(K)"),
    "last_page_tokens_off_by_one": ("return min(PAGE_TOKENS, L - j * PAGE_TOKENS)",
                                    "return min(PAGE_TOKENS, L - j * PAGE_TOKENS + 1)"),
    "values_not_transposed": (".reshape(D, PAGE_TOKENS).T", ".reshape(PAGE_TOKENS, D)"),
    "attend_no_scale": ("logits = (K @ q[h * self.G + j]) / math.sqrt(self.D)", "logits = (K @ q[h * self.G + j])"),
    "attend_wrong_kv_head": ("logits = (K @ q[h * self.G + j])", "logits = (K @ q[j * self.Hkv + h])"),
    "append_skips_resident_copy": ("                if c != FREE:\n                    dst.append(self.pool[b * self.C + c])",
                                   "                if c == -12345:\n                    dst.append(self.pool[b * self.C + c])"),
    "append_slot_off_by_one": ("slot_tok = (int(req.lens[tail]) - 1) % PAGE_TOKENS",
                               "slot_tok = int(req.lens[tail]) % PAGE_TOKENS"),
    "append_never_new_partition": ("if req.n_parts == 0 or req.lens[tail] % PAGE_TOKENS == 0:",
                                   "if req.n_parts == 0:"),
    "retrieve_wrong_head": ("src = self.requests[b].host[h, page]",
                            "src = self.requests[b].host[0, page]"),
    "retrieve_copies_padding": ("dst = np.zeros(PAGE_ELEMS, np.uint16)", "dst = src.copy()"),
    # request turnover
    "release_order_reversed": ("for e in range(self.ndir):\n                s = self.directory[b, h, e]\n                if s != FREE:\n",
                               "for e in reversed(range(self.ndir)):\n                s = self.directory[b, h, e]\n                if s != FREE:\n"),
    "release_keeps_budget": ("self.budget[b] = self.C\n        self.requests[b] = None", "self.requests[b] = None"),
    "release_keeps_segment_entries": ("self.segments[s, :] = FREE\n                    self.seg_live[s] = 0",
                                      "self.seg_live[s] = 0"),
    "release_keeps_last_use": ("self.owner[b, :] = FREE\n        self.last_use[b, :] = FREE", "self.owner[b, :] = FREE"),
    "reindex_without_release": ("        self.release(b)\n        req = Request(", "        req = Request("),
    # step order
    "rewound_step_accepted": ("if t < self.last_t:", "if t < self.last_t - 10 ** 6:"),
}


def _mutant(old: str, new: str) -> types.ModuleType:
    src = inspect.getsource(om)
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("spin_oracle_mutant")
    exec(compile(src.replace(old, new), "spin_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, MemoryError, ValueError, KeyError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects mutation {name}"
