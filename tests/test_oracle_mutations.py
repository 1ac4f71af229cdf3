"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case replaces one oracle function with a plausibly wrong version of it (a dropped term, a wrong
index or sign, a wrong rounding, a step in the wrong order), runs the pins that guard that part, and
requires at least one of them to fail.  A mistake no pin catches would mean the oracle's agreement with
the kernels proves less than it claims.  The planted code lives here and only here: the oracle itself is
never edited, and nothing else sees the replacement (pytest's monkeypatch undoes it after each case).
"""
import numpy as np
import pytest

from oracle import attention, codec, paged, step, wgemm

import test_oracle_alloc as T_alloc
import test_oracle_attention as T_attn
import test_oracle_codec as T_codec
import test_oracle_layers as T_layers
import test_oracle_paged as T_paged
import test_oracle_wgemm as T_wgemm

_real = {
    "softmax_attention": attention.softmax_attention,
    "dequant_rows": attention.dequant_rows,
    "e4m3_encode": codec.e4m3_encode,
    "tag_check": paged.tag_check,
    "gather": paged.gather,
    "append": paged.append,
    "quantize_w4": wgemm.quantize_w4,
}


# ----------------------------------------------------------------------------- the planted mistakes

def gqa_interleaved(mp):
    """Query head h reads KV head h % Hkv instead of h // (Hq / Hkv)."""
    def bad(q_r, k_rows, v_rows, num_kv_heads, sm_scale):
        out = np.empty((q_r.shape[0], v_rows.shape[2]))
        for h in range(q_r.shape[0]):
            g = h % num_kv_heads
            out[h] = _real["softmax_attention"](q_r[h:h + 1], k_rows[:, g, :], v_rows[:, g, :], sm_scale)[0]
        return out
    mp.setattr(attention, "request_attention", bad)


def dropped_softmax_scale(mp):
    mp.setattr(attention, "softmax_attention", lambda q, k, v, sm: _real["softmax_attention"](q, k, v, 1.0))


def scale_not_applied_on_read(mp):
    """The FP8 cache decoded without multiplying by its tensor scale."""
    mp.setattr(attention, "dequant_rows",
               lambda c, dtype, s: codec.e4m3_decode(c) if dtype == "fp8" else codec.f64_from_bf16(c))


def context_one_short(mp):
    """Attention over [0, L - 1) instead of [0, L) (the token written this step left out)."""
    mp.setattr(paged, "gather", lambda k, v, pt, r, n: _real["gather"](k, v, pt, r, max(n - 1, 1)))


def latent_values_from_the_tail(mp):
    """Latent cache: values taken from the last Dv dims of the vector instead of the first."""
    def bad(q, k, v, sm):
        if v.shape[1] < k.shape[1] and np.array_equal(v, k[:, :v.shape[1]]):
            v = k[:, k.shape[1] - v.shape[1]:]
        return _real["softmax_attention"](q, k, v, sm)
    mp.setattr(attention, "softmax_attention", bad)


def e4m3_round_down(mp):
    """Truncation toward zero instead of round to nearest even (|p| below 448)."""
    def bad(p):
        p = np.asarray(p, dtype=np.float64)
        c = _real["e4m3_encode"](p)
        mag = np.abs(np.nan_to_num(p))
        dec = np.abs(codec.e4m3_decode(c & 0x7F))
        over = (dec > mag) & (mag <= codec.E4M3_MAX) & ((c & 0x7F) > 0)
        return np.where(over, c - 1, c).astype(np.uint8)
    mp.setattr(codec, "e4m3_encode", bad)


def e4m3_ties_away_from_zero(mp):
    """Ties rounded away from zero instead of to even."""
    def bad(p):
        p = np.asarray(p, dtype=np.float64)
        c = _real["e4m3_encode"](p)
        mag = np.abs(np.nan_to_num(p))
        lo = np.abs(codec.e4m3_decode(c & 0x7F))
        up = np.abs(codec.e4m3_decode(np.minimum((c & 0x7F) + 1, 0x7E)))
        tie = (up > lo) & (mag - lo == up - mag) & (mag <= codec.E4M3_MAX)
        return np.where(tie, c + 1, c).astype(np.uint8)
    mp.setattr(codec, "e4m3_encode", bad)


def e4m3_overflow_to_nan(mp):
    """Magnitudes above 448 encoded as NaN instead of saturating."""
    def bad(p):
        p = np.asarray(p, dtype=np.float64)
        c = _real["e4m3_encode"](p)
        return np.where(np.abs(p) > codec.E4M3_MAX, c | 0x7F, c).astype(np.uint8)
    mp.setattr(codec, "e4m3_encode", bad)


def e4m3_decode_bias_8(mp):
    """Exponent bias 8 instead of 7."""
    real = codec.e4m3_decode
    mp.setattr(codec, "e4m3_decode", lambda c: real(c) * 0.5)


def bf16_truncates(mp):
    """float32 -> bfloat16 by dropping the low bits instead of rounding to nearest even."""
    mp.setattr(codec, "bf16_from_f32",
               lambda x: (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16))


def absmax_without_abs(mp):
    """The scale taken from max(x) instead of max|x|."""
    def bad(x):
        a = codec.f32_from_bf16(np.asarray(x).ravel())
        a = a[~np.isnan(a)]
        return np.float32(a.max() if a.size else 0).view(np.uint32)
    mp.setattr(codec, "absmax_bits", bad)


def tag_check_misses_last_page(mp):
    """The last used page-table entry is not checked."""
    def bad(page_tags, page_table, expected, ctx_lens, page_size):
        lens = np.asarray(ctx_lens).copy()
        lens = np.where(lens > page_size, ((lens - 1) // page_size) * page_size, lens)
        f = _real["tag_check"](page_tags, page_table, expected, lens, page_size)
        # keep the length test of the full context
        need = (np.asarray(ctx_lens) + page_size - 1) // page_size
        return f | np.where(need > page_table.shape[1], paged.FLAG_BAD_PAGE, 0).astype(np.uint32)
    mp.setattr(paged, "tag_check", bad)


def append_to_next_slot(mp):
    """A token written one slot past its position (pos % S + 1)."""
    def bad(k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table, flags=None):
        S = k_pool.shape[2]
        pos = np.asarray(tok_pos, dtype=np.int64)
        shifted = (pos // S) * S + (pos % S + 1) % S
        return _real["append"](k_pool, v_pool, k_new, v_new, tok_req, shifted, page_table, flags)
    mp.setattr(paged, "append", bad)


def step_appends_before_the_check(mp):
    """The step writes every token before the check (flags ignored by the write)."""
    def bad_append(k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table, flags=None):
        return _real["append"](k_pool, v_pool, k_new, v_new, tok_req, tok_pos, page_table, None)
    mp.setattr(paged, "append", bad_append)


def kv_bytes_without_v(mp):
    """The KV-size formula missing its factor 2 (K and V)."""
    mp.setattr(paged, "kv_bytes", lambda req, tok, lay, h, d, b: req * tok * lay * h * d * b)


def tag_bumped_on_free(mp):
    """The allocator bumps a page's tag when the page is freed instead of when it is handed out."""
    def alloc(self, n):
        if n > len(self.free_list):
            return self.NOSPACE
        pages = [self.free_list.pop() for _ in range(n)]
        for p in pages:
            self.in_use[p] = True
        return np.array(pages, dtype=np.int32), self.tags[pages].copy()

    real_free = paged.PageAllocator.free

    def free(self, pages):
        st = real_free(self, pages)
        if st is None:
            for p in pages:
                self.tags[int(p)] = np.uint32((int(self.tags[int(p)]) + 1) % 2 ** 32)
        return st
    mp.setattr(paged.PageAllocator, "alloc", alloc)
    mp.setattr(paged.PageAllocator, "free", free)


def w4_ties_away_from_zero(mp):
    """INT4 codes rounded half away from zero instead of half to even."""
    def bad(w_bits):
        wg = wgemm._groups(w_bits)
        s = wgemm._group_scale(wg, wgemm.INT4_MAX)
        prod = (wg * wgemm._inv(s)[:, :, None]).astype(np.float32).astype(np.float64)
        q = np.clip(np.sign(prod) * np.floor(np.abs(prod) + 0.5), -8, 7).astype(np.int8)
        return q.reshape(wg.shape[0], -1), s
    mp.setattr(wgemm, "quantize_w4", bad)


def w4_scale_over_8(mp):
    """INT4 scale max|w| / 8 instead of max|w| / 7."""
    mp.setattr(wgemm, "INT4_MAX", 8.0)


def w4_dequant_without_scale(mp):
    mp.setattr(wgemm, "dequant_w4", lambda q, s: q.astype(np.float64))


MUTANTS = {
    "gqa_interleaved": (gqa_interleaved, [T_attn.test_gqa_group_mapping_against_single_head_runs,
                                          lambda: T_attn.test_brute_force_tiny_shapes("fp8")]),
    "dropped_softmax_scale": (dropped_softmax_scale, [T_attn.test_two_token_closed_form,
                                                      lambda: T_attn.test_brute_force_tiny_shapes("bf16")]),
    "scale_not_applied_on_read": (scale_not_applied_on_read,
                                  [lambda: T_attn.test_single_token_returns_dequantised_value("fp8"),
                                   lambda: T_attn.test_brute_force_tiny_shapes("fp8")]),
    "context_one_short": (context_one_short, [lambda: T_attn.test_brute_force_tiny_shapes("bf16"),
                                              lambda: T_attn.test_equal_keys_give_mean_of_values("bf16")]),
    "latent_values_from_the_tail": (latent_values_from_the_tail,
                                    [lambda: T_attn.test_brute_force_latent_tiny_shapes("bf16"),
                                     T_attn.test_latent_matches_gqa_formula]),
    "e4m3_round_down": (e4m3_round_down, [lambda: T_codec.test_encode_brute_force_all_bf16(1.0),
                                          T_codec.test_encode_against_torch_in_range]),
    "e4m3_ties_away_from_zero": (e4m3_ties_away_from_zero,
                                 [lambda: T_codec.test_encode_brute_force_all_bf16(1.0)]),
    "e4m3_overflow_to_nan": (e4m3_overflow_to_nan, [T_codec.test_encode_saturation_and_specials]),
    "e4m3_decode_bias_8": (e4m3_decode_bias_8, [T_codec.test_decode_anchor_table,
                                                T_codec.test_decode_all_256_against_torch]),
    "bf16_truncates": (bf16_truncates, [T_codec.test_bf16_rne_against_torch]),
    "absmax_without_abs": (absmax_without_abs, [T_codec.test_scale_calibration]),
    "tag_check_misses_last_page": (tag_check_misses_last_page, [T_paged.test_tag_check_every_position_detected]),
    "append_to_next_slot": (append_to_next_slot, [T_paged.test_append_writes_exactly_the_addressed_elements]),
    "step_appends_before_the_check": (step_appends_before_the_check,
                                      [T_attn.test_decode_step_order_check_before_append,
                                       lambda: T_layers.test_stale_request_untouched_in_every_layer("fp8")]),
    "kv_bytes_without_v": (kv_bytes_without_v, [T_paged.test_kv_bytes_formula_and_capacity_doubling]),
    "tag_bumped_on_free": (tag_bumped_on_free, [T_alloc.test_fresh_allocator_hands_out_pages_in_order_with_bumped_tags,
                                                T_alloc.test_reallocation_changes_the_tag_and_reuses_last_freed_first]),
    "w4_ties_away_from_zero": (w4_ties_away_from_zero, [T_wgemm.test_int4_exact_multiples_and_ties]),
    "w4_scale_over_8": (w4_scale_over_8, [T_wgemm.test_int4_exact_multiples_and_ties,
                                          T_wgemm.test_int4_matches_torch_rounding]),
    "w4_dequant_without_scale": (w4_dequant_without_scale, [T_wgemm.test_gemm_one_hot_and_brute_force]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_pass_on_the_oracle_as_written(name):
    """The same pins all pass without the planted mistake (so a failure below is the mistake's)."""
    for pin in MUTANTS[name][1]:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    plant, pins = MUTANTS[name]
    plant(monkeypatch)
    failed = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed.append(pin)
    assert failed, f"no pin caught the planted mistake {name!r}"


def test_step_module_sees_the_patched_parts(monkeypatch):
    """The step composes the oracle's parts by module attribute, so a planted part is the one it runs."""
    seen = []
    monkeypatch.setattr(paged, "tag_check", lambda *a, **k: seen.append(1) or _real["tag_check"](*a, **k))
    T_attn.test_decode_step_order_check_before_append()
    assert seen and step.paged is paged
