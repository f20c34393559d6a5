"""The run-time tuning table (host side, CPU): parsing, precedence over the built-in table, fit
checks, clearing; and the autotuner's table output."""
import os

import pytest

import quantized_gemm_prepacked_amd as hq
from quantized_gemm_prepacked_amd import autotune


@pytest.fixture(autouse=True)
def _clear_table():
    hq.hq_load_tuning_table(None)
    yield
    hq.hq_load_tuning_table(None)


def _write(tmp_path, text):
    p = tmp_path / "table.txt"
    p.write_text(text)
    return str(p)


def test_entries_take_precedence_by_max_m(tmp_path):
    d = hq.DESC_W4A16_ASYM
    builtin = [hq.hq_gemm_plan(d, M, 14336, 4096) for M in (1, 16, 128, 8192)]
    builtin_k = hq.hq_gemm_plan(d, 1, 14336, 8192)
    hq.hq_load_tuning_table(_write(tmp_path, "# comment\nwna16 1 14336 4096 16 0 13 -1\n"
                                             "wna16 1 14336 4096 2000 1 0 1  # tiled\n"))
    assert hq.hq_gemm_plan(d, 1, 14336, 4096)[:2] == (0, 13)
    assert hq.hq_gemm_plan(d, 16, 14336, 4096)[:2] == (0, 13)
    assert hq.hq_gemm_plan(d, 128, 14336, 4096) == (1, 0, 1)
    assert hq.hq_gemm_plan(d, 8192, 14336, 4096) == builtin[3]        # past every max_m
    assert hq.hq_gemm_plan(hq.DESC_W4A16_SYM, 1, 14336, 4096) == builtin[0]   # other asym
    assert hq.hq_gemm_plan(d, 1, 14336, 8192) == builtin_k                  # other K
    hq.hq_load_tuning_table(None)
    assert [hq.hq_gemm_plan(d, M, 14336, 4096) for M in (1, 16, 128, 8192)] == builtin


def test_forced_skinny_split_and_unfit_entries(tmp_path):
    hq.hq_load_tuning_table(_write(tmp_path, "w8a8 0 8192 8192 64 0 1 4\n"
                                             "w4a8 0 4096 7168 64 1 0 1\n"))   # tiled cfg 0 needs N % 128
    assert hq.hq_gemm_plan(hq.DESC_W8A8, 32, 8192, 8192) == (0, 1, 4)
    # an entry naming a configuration that does not fit the shape is ignored: N = 4096 fits
    # tiled cfg 0, so this one is used; with N = 4112 (257 tiles) it would not be
    assert hq.hq_gemm_plan(hq.DESC_W4A8_MXFP4, 32, 4096, 7168)[0] == 1


def test_every_family_name_parses(tmp_path):
    lines = [f"{fam} {asym} 256 1024 8 0 2 -1" for _, (_, fam, asym) in autotune.FORMATS.items()]
    hq.hq_load_tuning_table(_write(tmp_path, "\n".join(lines) + "\n"))
    for fmt, (desc, _, _) in autotune.FORMATS.items():
        assert hq.hq_gemm_plan(desc, 4, 256, 1024)[:2] == (0, 2), fmt


@pytest.mark.parametrize("bad", ["wna16 1 14336 4096 16 0\n", "int3 0 256 256 8 0 0 1\n",
                                 "wna16 1 14336 4096 16 7 0 1\n", "wna16 1 14336 4096 16 0 0 0\n",
                                 "wna16 1 14336 4096 16 0 0 1 extra\n"])
def test_malformed_tables_fail_and_keep_the_old_one(tmp_path, bad):
    hq.hq_load_tuning_table(_write(tmp_path, "wna16 1 14336 4096 16 0 13 -1\n"))
    p = tmp_path / "bad.txt"
    p.write_text(bad)
    with pytest.raises(hq.HQError):
        hq.hq_load_tuning_table(str(p))
    assert hq.hq_gemm_plan(hq.DESC_W4A16_ASYM, 1, 14336, 4096)[:2] == (0, 13)
    with pytest.raises(hq.HQError):
        hq.hq_load_tuning_table(str(tmp_path / "missing.txt"))


def test_autotune_table_lines_cover_m_ranges(tmp_path):
    res = [dict(M=1, kind=0, cfg=28, split=1, us=9.6, default_us=9.8, default=(0, 28, 1)),
           dict(M=128, kind=2, cfg=2, split=1, us=39.0, default_us=39.3, default=(2, 2, 1)),
           dict(M=16, kind=0, cfg=13, split=-1, us=10.1, default_us=10.3, default=(0, 28, 1))]
    lines = autotune.table_lines("w4a16a", 14336, 4096, res)
    assert [ln.split("#")[0].split() for ln in lines] == [
        ["wna16", "1", "14336", "4096", "4", "0", "28", "1"],
        ["wna16", "1", "14336", "4096", "45", "0", "13", "-1"],
        ["wna16", "1", "14336", "4096", str(1 << 40), "2", "2", "1"]]
    hq.hq_load_tuning_table(_write(tmp_path, "\n".join(lines) + "\n"))
    d = hq.DESC_W4A16_ASYM
    assert hq.hq_gemm_plan(d, 4, 14336, 4096)[:2] == (0, 28)
    assert hq.hq_gemm_plan(d, 5, 14336, 4096)[:2] == (0, 13)
    assert hq.hq_gemm_plan(d, 46, 14336, 4096)[:2] == (2, 2)


def test_batch_invariant_plan_is_fixed_and_ignores_tables(tmp_path):
    inv = hq.with_flags(hq.DESC_W4A16_ASYM, hq.HQ_COMPUTE_BATCH_INVARIANT)
    plans = {hq.hq_gemm_plan(inv, M, 14336, 4096) for M in (1, 16, 128, 1024, 8192)}
    assert len(plans) == 1 and next(iter(plans))[0] == 0 and next(iter(plans))[2] == 1
    hq.hq_load_tuning_table(_write(tmp_path, "wna16 1 14336 4096 16 0 13 -1\n"))
    assert hq.hq_gemm_plan(inv, 1, 14336, 4096) in plans
    assert hq.hq_moe_block_m(hq.with_flags(hq.DESC_W4A16_SYM, hq.HQ_COMPUTE_BATCH_INVARIANT), 4096, 8, 256, 4096, 7168) == 32
    bad = hq.with_flags(hq.DESC_W4A16_ASYM, 6)
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(bad, 1, 14336, 4096)
