"""Pin: the Q8G64 row size and the capacity arithmetic printed on the offload page."""
import json
import os

import pytest

from tests.oracle_util import unit

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "capacity.json")))
UNIT = {"MiB": 2 ** 20, "GiB": 2 ** 30, "TiB": 2 ** 40}


def test_row_is_656_bytes_in_the_oracle():
    u = unit(max_positions=4)
    r = GOLD["row"]
    assert r["latent_bytes"] + r["scale_bytes"] + r["rope_bytes"] == r["total_bytes"] == 656
    assert u.row_bytes == r["total_bytes"]


@pytest.mark.parametrize("row", GOLD["table"], ids=lambda r: r["what"])
def test_capacity_table(row):
    u = unit(max_positions=4)
    b = row["tokens"] * row["layers"] * row["copies"] * u.row_bytes
    assert round(b / UNIT[row["unit"]], row["digits"]) == pytest.approx(row["printed"], abs=0)


def test_per_token_exchange_reduction():
    e = GOLD["exchange"]
    assert e["f32_bytes_per_token_layer"] == (512 + 64) * 4
    assert round(100 * (1 - e["q8g64_bytes"] / e["f32_bytes_per_token_layer"]), 1) == e["printed_reduction_percent"]
