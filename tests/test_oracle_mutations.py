"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case monkeypatches one plausible slip into the oracle and re-runs a pin
that should then fail: a transposed grouping, a slot off by one, a dropped
softmax scale, a wrong e5m2 exponent bias, a window one position too wide,
per-channel scales read with the dims reversed, a mixed-granularity V read
with the K channel scales, a radix-tree partial match without its copy, an
eviction of the most recently used leaf, an eviction of an inner block, a
shared prefix read through the sequences' own tables, a shared prefix read
past a short context, a shared/own boundary one position off.
"""

import numpy as np
import pytest

import oracle.attention as att
import oracle.codecs as codecs
from tests import test_oracle_attention as ta
from tests import test_oracle_codecs as tc
from tests import test_oracle_paging as tp
from tests import test_oracle_int8_scales as ti
from tests import test_oracle_window as tw
from tests import test_oracle_shared_prefix as tsp
from oracle import layout


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_wrong_group_mapping_is_caught(monkeypatch):
    orig = att.attend

    def attend_bad(q, K, V, scale):
        hq = q.shape[0]
        hkv = K.shape[1]
        perm = np.arange(hq).reshape(hkv, hq // hkv).T.ravel()   # h % Hkv grouping
        return orig(q[perm], K, V, scale)[np.argsort(perm)]
    monkeypatch.setattr(att, "attend", attend_bad)
    assert _fails(ta.test_tiny_config_matches_sdpa)


def test_slot_off_by_one_is_caught(monkeypatch):
    # the element-by-element gather follows slot_of; the whole-tile gather must
    # equal it, so a slot slip shows as a mismatch between the two
    def slot_bad(row, pos, B):
        pos = np.asarray(pos, dtype=np.int64)
        row = np.asarray(row, dtype=np.int64)
        return row[pos // B] * B + (pos + 1) % B
    monkeypatch.setattr(att, "slot_of", slot_bad)
    assert _fails(lambda: tp.test_tile_gather_equals_slot_gather(layout.KV_BF16, 16, 64))


def test_token_shift_in_tile_read_is_caught(monkeypatch):
    orig = att.layout_k_tokens
    monkeypatch.setattr(att, "layout_k_tokens", lambda *a: np.roll(orig(*a), 1, axis=0))
    assert _fails(ta.test_tiny_config_matches_sdpa)


def test_dropped_scale_is_caught(monkeypatch):
    orig = att.attend
    monkeypatch.setattr(att, "attend", lambda q, K, V, s: orig(q, K, V, 1.0))
    assert _fails(lambda: ta.test_random_small_cases_match_sdpa(3))


def test_wrong_e5m2_bias_is_caught(monkeypatch):
    orig = codecs.e5m2_decode
    monkeypatch.setattr(codecs, "e5m2_decode", lambda c: orig(c) * 2.0)
    assert _fails(tc.test_e5m2_decode_matches_binary16_high_byte)


def test_window_off_by_one_is_caught(monkeypatch):
    orig = att.window_start
    monkeypatch.setattr(att, "window_start", lambda ctx, w: max(orig(ctx, w) - 1, 0))
    assert _fails(lambda: tw.test_window_matches_masked_sdpa(3))


def test_reversed_channel_scales_are_caught(monkeypatch):
    def bad(p, layer, head, d):
        return (np.asarray(layer, dtype=np.int64) * p.num_kv_heads + head) * p.head_dim + (p.head_dim - 1 - d)
    monkeypatch.setattr(att, "channel_scale_offset", bad)
    assert _fails(lambda: ti.test_cache_write_then_gathers_read_code_times_scale(layout.KV_INT8_CHANNEL))


def test_swapped_int4_nibble_halves_are_caught(monkeypatch):
    from tests import test_oracle_int4 as t4
    real = layout.int4_v_nibble

    def bad(p, layer, block, head, t, d):
        return real(p, layer, block, head, t, d) ^ 1      # low and high nibble of each byte swapped
    monkeypatch.setattr(layout, "int4_v_nibble", bad)
    assert _fails(lambda: t4.test_each_v_byte_holds_one_token_and_each_k_word_one_mfma_slot(16, 128)) or \
        _fails(lambda: t4.test_tile_unpack_equals_element_reads(16, 128))


def test_int4_offset_of_seven_is_caught(monkeypatch):
    from tests import test_oracle_int4 as t4
    real = codecs.int4_encode
    monkeypatch.setattr(codecs, "int4_encode", lambda x, s: np.clip(real(x, s), -7, 6).astype(np.int8))
    assert _fails(t4.test_bound_saturation_and_zero_scale)


def test_causal_limit_off_by_one_is_caught(monkeypatch):
    # each query also attends to the key right after its own position
    from tests import test_oracle_prefill as tpf
    real = att.attend

    def attend_one_more(q, K, V, scale):
        return real(q, K, V, scale)

    def bad(q_bits, img, layer, bt, ctx, qs, scale, ks=1.0, vs=1.0):
        q_bits = np.asarray(q_bits, dtype=np.uint16)
        out = np.zeros(q_bits.shape, dtype=np.float64)
        for s in range(len(ctx)):
            c, n = int(ctx[s]), int(qs[s + 1] - qs[s])
            K, V = att.gather_kv(img, layer, bt[s], c, ks, vs)
            q = codecs.bf16_bits_to_f64(q_bits[qs[s]:qs[s + 1]])
            for k in range(n):
                pos = c - n + k
                out[qs[s] + k] = attend_one_more(q[k], K[:pos + 2], V[:pos + 2], scale)
        return out
    monkeypatch.setattr(att, "paged_prefill", bad)
    assert _fails(lambda: tpf.test_whole_prompt_equals_matrix_causal_attention(1))


def test_mixed_granularity_v_read_with_a_k_scale_is_caught(monkeypatch):
    # K per channel, V per tensor: a dequantiser that takes V's scale from the
    # K channel scales (the per-channel rule applied to both) must fail the
    # pin tying the mixed type to INT8 per channel with uniform V scales
    orig = att._dequant_fixed_scales

    def bad(p, img, layer, kraw, vraw, k_scale, v_scale):
        k, v = orig(p, img, layer, kraw, vraw, k_scale, v_scale)
        if p.kv_dtype == layout.KV_INT8_KCHANNEL_VTENSOR:
            co = layout.channel_scale_offset(p, layer, np.arange(p.num_kv_heads)[:, None],
                                             np.arange(p.head_dim)[None, :])
            v = vraw.astype(np.float64) * img.k_scale[co].astype(np.float64)[None]
        return k, v
    monkeypatch.setattr(att, "_dequant_fixed_scales", bad)
    assert _fails(ti.test_int8_per_channel_with_equal_v_scales_is_the_mixed_granularity)
    assert _fails(ti.test_mixed_one_token_context_returns_v_code_times_v_scale)


def test_radix_partial_match_without_its_copy_is_caught(monkeypatch):
    from oracle.block_manager import BlockManagerModel
    from tests import test_oracle_radix as tr
    orig = BlockManagerModel.add_seq_radix

    def no_copy(self, seq, tokens):
        st, cached, pair = orig(self, seq, tokens)
        return st, cached, None                  # the copy of the partly matched block is lost
    monkeypatch.setattr(BlockManagerModel, "add_seq_radix", no_copy)
    assert _fails(lambda: tr.test_pages_example_shares_six_tokens(4))


def test_radix_most_recently_used_eviction_is_caught(monkeypatch):
    from oracle.block_manager import BlockManagerModel
    from tests import test_oracle_radix as tr

    def evict_mru(self):
        leaves = [b for b in self.node_parent if self.ref[b] == 0 and not self.children[b]]
        b = max(leaves, key=lambda x: (self.last_use[x], self.node_depth[x], -x))
        self.children[self.node_parent[b]].remove(b)
        for d in (self.node_parent, self.node_tokens, self.node_depth, self.children, self.last_use):
            del d[b]
        return b
    monkeypatch.setattr(BlockManagerModel, "_evict", evict_mru)
    assert _fails(tr.test_lru_leaves_go_first_and_shared_prefix_survives)


def test_radix_eviction_of_an_inner_block_is_caught(monkeypatch):
    from oracle.block_manager import BlockManagerModel
    from tests import test_oracle_radix as tr

    def evict_any(self):
        # the leaf condition forgotten: the shallowest idle block goes, and
        # its cached children keep pointing at a block that now holds
        # another sequence's tokens
        idle = [b for b in self.node_parent if self.ref[b] == 0]
        b = min(idle, key=lambda x: (self.last_use[x], self.node_depth[x], x))
        self.children[self.node_parent[b]].remove(b)
        for d in (self.node_parent, self.node_tokens, self.node_depth, self.last_use):
            del d[b]
        return b
    monkeypatch.setattr(BlockManagerModel, "_evict", evict_any)
    assert _fails(lambda: [tr.test_random_walk_under_eviction(2, s) for s in range(4)])


def test_shared_prefix_read_through_own_tables_is_caught(monkeypatch):
    monkeypatch.setattr(att, "shared_prefix_bounds", lambda ctx, P: (0, 0))
    assert _fails(lambda: tsp.test_shared_prefix_matches_sdpa_on_the_token_lists(0))


def test_shared_prefix_past_a_short_context_is_caught(monkeypatch):
    monkeypatch.setattr(att, "shared_prefix_bounds", lambda ctx, P: (P, P))
    assert _fails(lambda: tsp.test_shared_prefix_equals_decode_of_materialised_copies(layout.KV_BF16))


def test_shared_prefix_boundary_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(att, "shared_prefix_bounds", lambda ctx, P: (max(min(ctx, P) - 1, 0), max(P - 1, 0)))
    assert _fails(lambda: tsp.test_shared_prefix_matches_sdpa_on_the_token_lists(1))
