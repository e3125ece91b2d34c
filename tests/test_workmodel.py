"""The algorithmic byte model used for every roofline figure, pinned to the
numbers the decode page prints ("feat(kda): add packed-input CuTe decode
kernel", sections "Benchmark results" and "DRAM utilization"; fixture in
tests/golden/decode_dram_utilization.txt)."""
import os

from gated_delta_rule_step_amd import workmodel as wm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_dram_utilization.txt")


def _golden():
    rows, facts = [], {}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        if len(line) == 5:
            rows.append((int(line[0]), *map(float, line[1:])))
        else:
            facts[line[0]] = (float(line[1]), line[2])
    return rows, facts


def test_decode_bytes_reproduce_printed_bandwidth():
    """Compulsory bytes / printed median time, rounded as printed, gives the
    printed TB/s at every batch for both kernel variants."""
    rows, _ = _golden()
    assert len(rows) == 4
    for B, us_prev, tb_prev, us_this, tb_this in rows:
        nbytes = wm.decode_bytes(B, 0)
        assert round(nbytes / (us_prev * 1e-6) / 1e12, 2) == tb_prev, (B, "prev")
        assert round(nbytes / (us_this * 1e-6) / 1e12, 2) == tb_this, (B, "this")


def test_decode_byte_components_match_printed_sizes():
    _, facts = _golden()
    H = 12
    round_trip = 2 * wm.SB * H
    assert round(round_trip / 1e3) == facts["state_round_trip_per_row"][0]
    assert int(512 * round_trip / 1e6) == facts["state_round_trip_B512"][0]
    assert round((wm.TOK_IN + wm.TOK_OUT) * H / 1e3) == facts["activations_per_row"][0]


def test_verify_and_prefill_bytes_closed_forms():
    """Verify and prefill byte counts against their per-unit sums written out."""
    H = 12
    per_row_bare_t8 = wm.SB * H + 8 * (wm.TOK_IN + wm.TOK_OUT + wm.RING_ROW) * H + 3 * wm.IDX
    assert per_row_bare_t8 == 614_604
    assert wm.verify_bytes(8, [0] * 512, [False] * 512) == 512 * 614_604
    # a folding row with 5 history rows adds 5 ring rows read and one state written
    assert wm.verify_bytes(8, [5], [True]) == 614_604 + 5 * wm.RING_ROW * H + wm.SB * H
    assert wm.prefill_bytes((3840, 3776, 3200, 3072), 64) == \
        13_888 * 64 * 1282 + 4 * 64 * 2 * wm.SB + 5 * wm.IDX


def test_chunk_flops_at_64():
    """9.13 MFLOP per full 64-token chunk and head for the chunkwise form."""
    assert abs(wm.chunk_flops(64) / 1e6 - 9.13) < 0.005
