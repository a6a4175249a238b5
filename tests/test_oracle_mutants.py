"""Plant plausible mistakes in copies of oracle.c (on the CPU) and check that
each one fails at least one of the oracle's pins.  This is what makes the pins
worth trusting: a dropped term, a wrong sign, index or operand anywhere in the
oracle shows up."""

import os

import pytest

import oracle
import pins

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("e4m3_exponent_bias", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    ("e4m3_subnormal_scale", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("e4m3_sign_dropped", "return sign ? -mag : mag;", "return mag;"),
    ("e4m3_nan_missing", "if (e == 15 && m == 7) return NAN;", ""),
    ("bf16_shift", "(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    ("block_index_wrong_divisor", "t / pb->BS]", "t / (pb->BS + 1)]"),
    ("slot_off_by_one", "orc_kv(pb, 0, blk, t % pb->BS, h, d)", "orc_kv(pb, 0, blk, (t + 1) % pb->BS, h, d)"),
    ("cache_head_ignored", "return (blk * Hkv + h) * BS + slot;", "return (blk * Hkv + 0) * BS + slot;"),
    ("scale_field_ignored", "* 2 + field) * pb->BS + slot]", "* 2 + 0) * pb->BS + slot]"),
    ("scale_slot_ignored", "* 2 + field) * pb->BS + slot]", "* 2 + field) * pb->BS + 0]"),
    ("q_row_group_ignored", "(int64_t)h * pb->QG + g) * pb->D", "(int64_t)h * pb->QG + 0) * pb->D"),
    ("softmax_scale_dropped", "*x = pb->scale * dot;", "*x = dot;"),
    ("no_normalisation", "for (int d = 0; d < pb->D; ++d) o[d] /= l;", ""),
    ("weights_not_exponentiated", "double w = exp(xbuf[t - t0] - m);", "double w = xbuf[t - t0] - m;"),
    ("k_operand_is_v", "orc_kv(pb, 0, blk, t % pb->BS, h, d)", "orc_kv(pb, 1, blk, t % pb->BS, h, d)"),
    ("partition_end_off_by_one", "int t0 = p * E, t1 = (p + 1) * E < L ? (p + 1) * E : L;",
     "int t0 = p * E, t1 = (p + 1) * E < L ? (p + 1) * E - 1 : L;"),
    ("merge_weight_no_exp", "double w = l[r] * exp(m[r] - M);", "double w = l[r];"),
    ("merge_weight_no_l", "double w = l[r] * exp(m[r] - M);", "double w = exp(m[r] - M);"),
    ("merge_first_partition_only", "for (int p = 0; p < live; ++p) {\n          int64_t r",
     "for (int p = 0; p < 1; ++p) {\n          int64_t r"),
    ("merge_no_division", "for (int d = 0; d < D; ++d) dst[d] /= W;", ""),
    ("enc_ties_to_odd", "(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    ("enc_search_range_short", "for (int c = 0; c <= 0x7E; ++c) {", "for (int c = 0; c < 0x7E; ++c) {"),
    ("enc_sign_dropped", "(signbit(x) ? 0x80 : 0x00) | best", "best"),
    ("writer_fnuz_max", "float s = absmax / 448.0f;", "float s = absmax / 240.0f;"),
    ("writer_offset_wrong", "int blk = slot / BS, off = slot % BS;", "int blk = slot / BS, off = 0;"),
    ("writer_scale_field_swapped", "kv_scales[(((int64_t)blk * Hkv + h) * 2 + field) * BS + off] = s;",
     "kv_scales[(((int64_t)blk * Hkv + h) * 2 + (1 - field)) * BS + off] = s;"),
    ("writer_ignores_skip", "if (slot < 0) continue;", "if (slot < 0) slot = 0;"),
    ("f16_exponent_bias", "ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    ("f16_subnormal_scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("tq4_nibble_order", "int idx = (d & 1) ? byte >> 4 : byte & 0xF;",
     "int idx = (d & 1) ? byte & 0xF : byte >> 4;"),
    ("tq4_kv_regions_swapped", "row[(field == 0 ? 0 : pb->D / 2) + d / 2]",
     "row[(field == 0 ? pb->D / 2 : 0) + d / 2]"),
    ("tq4_norm_field", "return (double)pb->centroids[idx] * orc_dec_f16(f[0]);",
     "return (double)pb->centroids[idx] * orc_dec_f16(f[1]);"),
    ("tq4_zero_point_dropped", "return (double)idx * orc_dec_f16(f[1]) + orc_dec_f16(f[2]);",
     "return (double)idx * orc_dec_f16(f[1]);"),
    ("tq4_centroid_off_by_one", "pb->centroids[idx]", "pb->centroids[(idx + 1) & 15]"),
    ("tq4_meta_head_stride", "(int64_t)h * 3 * pb->BS * 2;", "(int64_t)h * 2 * pb->BS * 2;"),
    ("tq4_rows_slot_major", "orc_row(pb->layout, pb->Hkv, pb->BS, 0, h, slot)",
     "orc_row(ORC_LAYOUT_SLOT_MAJOR, pb->Hkv, pb->BS, 0, h, slot)"),
    # the slot-major row order (the page's data region) ignored everywhere, or in one reader
    ("layout_ignored", "if (layout == ORC_LAYOUT_SLOT_MAJOR) return (blk * BS + slot) * Hkv + h;", ""),
    ("slot_major_block_stride", "return (blk * BS + slot) * Hkv + h;", "return (blk * Hkv + slot) * Hkv + h;"),
    ("slot_major_head_and_slot_swapped", "return (blk * BS + slot) * Hkv + h;",
     "return (blk * BS + h) * Hkv + slot;"),
    ("tq4_layout_ignored", "orc_row(pb->layout, pb->Hkv, pb->BS, 0, h, slot)",
     "orc_row(ORC_LAYOUT_HEAD_MAJOR, pb->Hkv, pb->BS, 0, h, slot)"),
    ("fp8_layout_ignored", "orc_row(pb->layout, pb->Hkv, pb->BS, blk, h, slot)",
     "orc_row(ORC_LAYOUT_HEAD_MAJOR, pb->Hkv, pb->BS, blk, h, slot)"),
    ("writer_layout_ignored", "orc_row(layout, Hkv, BS, blk, h, off)",
     "orc_row(ORC_LAYOUT_HEAD_MAJOR, Hkv, BS, blk, h, off)"),
    # the partial triple's m_p in log2 units with a merge that matches: the merged result is
    # unchanged, only the partials' definition catches it
    ("partials_and_merge_log2_units",
     ("rc = orc_attend(&pb, s, h, g, t0, t1, xbuf, o + r * D, &m[r], &l[r]);",
      "double w = l[r] * exp(m[r] - M);"),
     ("rc = orc_attend(&pb, s, h, g, t0, t1, xbuf, o + r * D, &m[r], &l[r]); m[r] *= 1.4426950408889634;",
      "double w = l[r] * exp2(m[r] - M);")),
    # unnormalised partial outputs with a merge that does not weight by l_p
    ("partials_unnormalised_merge_without_l",
     ("for (int d = 0; d < pb->D; ++d) o[d] /= l;", "double w = l[r] * exp(m[r] - M);"),
     ("", "double w = exp(m[r] - M);")),
    ("tq4_block_stride", "(int64_t)pb->Hkv * 3 * pb->BS * 2;\n}", "(int64_t)pb->Hkv * 2 * pb->BS * 2;\n}"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    # a mutant is one replacement, or several applied together (tuples of sites)
    olds, news = (old, new) if isinstance(old, tuple) else ((old,), (new,))
    mutated = src
    for o_, n_ in zip(olds, news):
        assert mutated.count(o_) >= 1, f"mutation site for {name} not found in oracle.c"
        mutated = mutated.replace(o_, n_, 1)
    orc = oracle.build_variant(mutated, os.path.join(str(tmp_path), f"mut_{name}.so"))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # any failure of the pin counts as caught
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
