"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each: evidence that the pins fix every part of what the
oracle computes, not only its happy path."""

import pytest
import torch

import oracle.paged_attention as oracle_mod
from tests.oracle_pins import ALL_CHECKS

_orig = {name: getattr(oracle_mod, name) for name in
         ("kv_head_of", "token_location", "attend", "visible_keys", "merge_partitions",
          "kv_cache_write", "widen", "materialize")}


def _interleaved_groups(h, num_q_heads, num_kv_heads):
    return h % num_kv_heads


def _offset_off_by_one(t, table_row, block_size):
    pb, off = _orig["token_location"](t, table_row, block_size)
    return pb, (off + 1) % block_size


def _ignore_block_table(t, table_row, block_size):
    return (t // block_size).to(torch.int64), t % block_size


def _no_scale(q_vec, keys, values, scale):
    return _orig["attend"](q_vec, keys, values, 1.0)


def _mean_not_sum(q_vec, keys, values, scale):
    s = scale * (keys @ q_vec)
    w = torch.exp(s - s.max())
    return (w @ values) / w.numel()


def _keys_transposed_heads(q_vec, keys, values, scale):
    # values weighted by the softmax of the wrong operand order
    s = scale * (values @ q_vec)
    w = torch.exp(s - s.max())
    return (w @ values) / w.sum()


def _diagonal_masked(cached, row):
    return cached + row if cached + row > 0 else 1


def _top_left_mask(cached, row):
    return row + 1


def _merge_without_rescale(max_logits, exp_sums, partial_out, num_partitions):
    return _orig["merge_partitions"](torch.zeros_like(max_logits), exp_sums, partial_out, num_partitions)


def _write_swapped_index(key, value, slot_mapping, k_cache, v_cache):
    B = k_cache.shape[1]
    nb = k_cache.shape[0]
    remapped = torch.tensor([(s % nb) * B + (s // nb) % B if s >= 0 else s for s in slot_mapping.tolist()])
    return _orig["kv_cache_write"](key, value, remapped, k_cache, v_cache)


def _write_keeps_padding(key, value, slot_mapping, k_cache, v_cache):
    fixed = slot_mapping.clone()
    fixed[fixed < 0] = 0
    return _orig["kv_cache_write"](key, value, fixed, k_cache, v_cache)


def _narrow_to_fp32(x):
    return x.to(torch.float32).to(torch.float64)


def _materialize_one_block_short(cache, table_row, ctx):
    out = _orig["materialize"](cache, table_row, ctx)
    B = cache.shape[1]
    if ctx > B:
        out = out.clone()
        out[-1] = out[-1 - B]
    return out


MUTANTS = [
    ("kv_head_of", _interleaved_groups),
    ("token_location", _offset_off_by_one),
    ("token_location", _ignore_block_table),
    ("attend", _no_scale),
    ("attend", _mean_not_sum),
    ("attend", _keys_transposed_heads),
    ("visible_keys", _diagonal_masked),
    ("visible_keys", _top_left_mask),
    ("merge_partitions", _merge_without_rescale),
    ("kv_cache_write", _write_swapped_index),
    ("kv_cache_write", _write_keeps_padding),
    ("widen", _narrow_to_fp32),
    ("materialize", _materialize_one_block_short),
]


@pytest.mark.parametrize("attr,mutant", MUTANTS, ids=[m.__name__.lstrip("_") for _, m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, attr, mutant):
    monkeypatch.setattr(oracle_mod, attr, mutant)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(oracle_mod)
        except Exception as e:  # any failure (assertion, shape error) counts as caught
            caught.append((check.__name__, type(e).__name__))
            break
    assert caught, f"no pin caught the planted mistake in {attr}"
