"""Pins the oracle's cache accounting to the byte counts the pages print
(tests/golden/cache_accounting.json, every entry cited there)."""

import json
import os

import pytest

from oracle import mla

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_accounting.json")))

KiB, MiB, GiB = 1024, 1024 ** 2, 1024 ** 3


def test_elements_per_token():
    a, b = GOLD["elements_per_token"]
    assert mla.mla_cache_elems_per_token(a["d_c"], a["d_rope"]) == a["value"]
    assert mla.expanded_cache_elems_per_token(b["heads"], b["d_nope"], b["d_rope"], b["d_v"]) == b["value"]


def _active(entry):
    if "elems" in entry:
        return mla.cache_bytes(entry["tokens"], entry["elems"] * 2)
    if entry["kind"] == "latent":
        return mla.cache_bytes(entry["tokens"], mla.mla_bytes_per_token(512, 64))
    return mla.cache_bytes(entry["tokens"], mla.expanded_cache_elems_per_token(16) * 2)


@pytest.mark.parametrize("entry", GOLD["active_bytes_bf16"], ids=lambda e: e["what"])
def test_active_bytes(entry):
    assert _active(entry) == entry["value"]


@pytest.mark.parametrize("entry", GOLD["allocated_bytes_bf16_32_slots"], ids=lambda e: e["what"])
def test_allocated_bytes(entry):
    per_tok = (mla.mla_bytes_per_token(512, 64) if entry["kind"] == "latent"
               else mla.expanded_cache_elems_per_token(16) * 2)
    # the page's buffer holds 32 slots; 26 active tokens fit one 32-slot block
    assert mla.paged_allocated_bytes(entry["tokens"], per_tok, block=entry["slots"]) == entry["value"]


def test_ratios():
    naive = mla.cache_bytes(26, mla.expanded_cache_elems_per_token(16) * 2)
    absorb = mla.cache_bytes(26, mla.mla_bytes_per_token())
    r = GOLD["ratios"]
    # the page prints the repeating decimal cut off ("8.888888…"): compare the
    # exact ratio's digits by truncation, and the ratio itself as 80/9
    from fractions import Fraction
    ratio = Fraction(naive, absorb)
    assert ratio == Fraction(80, 9)
    assert str(int(ratio * 10**6) / 10**6) == r[0]["printed"]
    assert f"{100 * (1 - absorb / naive):.2f}%" == r[1]["printed"]


def test_bytes_per_token():
    e = GOLD["bytes_per_token_bf16"]
    eager = mla.expanded_cache_elems_per_token(16) * 2
    lat = mla.mla_bytes_per_token()
    assert eager == e[0]["value"] and lat == e[1]["value"]
    assert f"{eager / lat:.4f}" == e[2]["printed"]
    assert mla.mha_bytes_per_token(e[3]["n_h"], e[3]["d_h"]) == e[3]["value"]
    assert mla.mla_bytes_per_token(e[4]["d_c"], e[4]["d_r"]) == e[4]["value"]
    assert f"{e[3]['value'] / e[4]['value']:.1f}" == "56.9"


@pytest.mark.parametrize("row", GOLD["per_token_table_KB"], ids=lambda r: r["config"])
def test_per_token_table(row):
    mha = mla.mha_bytes_per_token(row["n_h"], row["d_h"])
    gqa = mla.gqa_bytes_per_token(row["n_kv"], row["d_h"])
    ml = mla.mla_bytes_per_token(row["d_c"], row["d_r"])
    assert f"{mha / KiB:.2f}" == row["MHA"]
    assert f"{gqa / KiB:.2f}" == row["GQA8"]
    assert f"{ml / KiB:.2f}" == row["MLA"]
    tok = 60 * 32 * 1024

    def gb(x):
        s = f"{x * tok / GiB:.2f}"
        return s.rstrip("0").rstrip(".")
    assert gb(mha) == row["MHA_60Lx32k_GB"]
    assert gb(gqa) == row["GQA_60Lx32k_GB"]
    assert gb(ml) == row["MLA_60Lx32k_GB"]


def _fmt_size(x):
    return f"{x / GiB:.2f} GB" if x >= GiB else f"{x / MiB:.2f} MB"


@pytest.mark.parametrize("row", GOLD["live_allocation_per_layer"], ids=lambda r: str(r["L"]))
def test_live_allocation(row):
    mha = mla.cache_bytes(row["L"], mla.mha_bytes_per_token(128, 128))
    ml = mla.cache_bytes(row["L"], mla.mla_bytes_per_token(512, 64))
    assert _fmt_size(mha) == row["MHA"]
    assert _fmt_size(ml) == row["MLA"]
    assert f"{mha / ml:.1f}" == row["ratio"]


@pytest.mark.parametrize("row", GOLD["bench_cache_column_MB"], ids=lambda r: str(r["prefill"]))
def test_bench_cache_column(row):
    L = row["prefill"] + row["decode"]
    mha = mla.cache_bytes(L, mla.mha_bytes_per_token(row["n_h"], row["d_h"]))
    ml = mla.cache_bytes(L, mla.mla_bytes_per_token(row["d_c"], row["d_r"]))
    assert f"{mha / MiB:.2f}" == row["MHA"]
    assert f"{ml / MiB:.2f}" == row["MLA"]


def test_planted_wrong_formula_is_caught():
    """A plausible slip (value cache counted with the rope width) must break a pin."""
    wrong = 16 * (128 + 64) * 2
    assert wrong * 26 * 2 != GOLD["active_bytes_bf16"][5]["value"]
