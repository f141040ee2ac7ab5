"""Pins for oracle.layout: hand bytes, bijections, round trips."""
import json
import os

import numpy as np
import pytest

from oracle import layout

HERE = os.path.dirname(__file__)
G = json.load(open(os.path.join(HERE, "golden", "layout_hand.json")))


def test_hand_pack():
    b = layout.pack_nibbles(np.array(G["pack"]["codes"], np.uint8))
    assert list(b) == G["pack"]["bytes"]


def test_nibbles_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    assert np.array_equal(layout.pack_nibbles(layout.unpack_nibbles(b)), b)


def test_record_sizes():
    rb = G["record_bytes"]
    assert layout.tq4_record_bytes(64) == rb["tq4_64"]
    assert layout.tq4_record_bytes(128) == rb["tq4_128"]
    assert layout.mxfp4_record_bytes(128) == rb["mxfp4_128"]
    assert layout.tq4_sections(128)["bytes"] == rb["tq4_128"]
    assert layout.mxfp4_sections(128)["bytes"] == rb["mxfp4_128"]


def test_hand_sections():
    sec = G["sections"]
    assert layout.tq4_sections(128) == sec["tq4_128"]
    assert layout.tq4_sections(64) == sec["tq4_64"]
    assert layout.tq4v2_sections(128) == sec["tq4v2_128"]
    assert layout.tq4v2_sections(64) == sec["tq4v2_64"]
    assert layout.mxfp4_sections(128) == sec["mxfp4_128"]
    # the large sections start on 128-byte lines; D = 128 records are whole lines
    for d in (64, 128):
        for s in (layout.tq4_sections(d), layout.tq4v2_sections(d)):
            assert s["vc"] % 128 == 0 and s["vm"] % 128 == 0
    for s in (layout.tq4_sections(128), layout.tq4v2_sections(128), layout.mxfp4_sections(128)):
        assert s["bytes"] % 128 == 0


def test_hand_offsets():
    for e in G["kc"]:
        assert int(layout.kc_offset(e["t"], e["p"], e["d"])) == e["off"]
    for e in G["vc"]:
        assert int(layout.vc_offset(e["t"], e["p"], e["d"])) == e["off"]
    for e in G["vm"]:
        so, mo = layout.vm_offsets(e["t"], e["gp"], e["d"])
        assert (int(so), int(mo)) == (e["scale"], e["min"])


@pytest.mark.parametrize("d", [64, 128])
def test_offset_maps_are_bijections(d):
    t = np.arange(16)[:, None]
    p = np.arange(d // 2)[None, :]
    for off in (layout.kc_offset(t, p, d), layout.vc_offset(t, p, d)):
        assert np.array_equal(np.sort(off.ravel()), np.arange(16 * d // 2))
    gp = np.arange(d // 32)[None, :]
    so, mo = layout.vm_offsets(t, gp, d)
    allb = np.concatenate([so.ravel(), so.ravel() + 1, mo.ravel(), mo.ravel() + 1])
    assert np.array_equal(np.sort(allb), np.arange(16 * (d // 32) * 4))
    if d == 128:
        assert np.array_equal(np.sort(layout.ks4_offset(t, gp).ravel()), np.arange(64))
        assert np.array_equal(np.sort(layout.vs4_offset(t, gp, d).ravel()), np.arange(64))


@pytest.mark.parametrize("d", [64, 128])
def test_tq4_write_read_round_trip(d):
    rng = np.random.default_rng(16)
    n = 16
    rec = np.zeros((n, layout.tq4_record_bytes(d)), np.uint8)
    rows = rng.permutation(16)
    kc = rng.integers(0, 16, (n, d)).astype(np.uint8)
    vc = rng.integers(0, 16, (n, d)).astype(np.uint8)
    ks = rng.standard_normal(n).astype(np.float16)
    sc = rng.standard_normal((n, d // 32)).astype(np.float16)
    mn = rng.standard_normal((n, d // 32)).astype(np.float16)
    # all 16 rows of one block, written together into one record
    one = np.zeros(rec.shape[1], np.uint8)
    layout.tq4_write_rows(one, np.zeros(n, np.int64), rows, d, kc, ks, vc, sc, mn)
    back = layout.tq4_read_block(one[None], d)
    for i in range(n):
        t = rows[i]
        assert np.array_equal(back["kcode"][0, t], kc[i])
        assert np.array_equal(back["vcode"][0, t], vc[i])
        assert back["kscale"][0, t].view(np.uint16) == ks[i].view(np.uint16)
        assert np.array_equal(back["vscale"][0, t].view(np.uint16), sc[i].view(np.uint16))
        assert np.array_equal(back["vmin"][0, t].view(np.uint16), mn[i].view(np.uint16))


def test_mxfp4_write_read_round_trip():
    rng = np.random.default_rng(17)
    d = 128
    rec = np.zeros((16, layout.mxfp4_record_bytes(d)), np.uint8)
    kc = rng.integers(0, 16, (16, d)).astype(np.uint8)
    vc = rng.integers(0, 16, (16, d)).astype(np.uint8)
    kx = rng.integers(-127, 128, (16, 4))
    vx = rng.integers(-127, 128, (16, 4))
    t = np.arange(16)
    one = np.zeros((16, rec.shape[1]), np.uint8)
    # row i goes to record i, token row i
    layout.mxfp4_write_rows(one.reshape(-1), t * rec.shape[1], t, d, kc, kx, vc, vx)
    back = layout.mxfp4_read_block(one, d)
    for i in range(16):
        assert np.array_equal(back["kcode"][i, i], kc[i])
        assert np.array_equal(back["vcode"][i, i], vc[i])
        assert np.array_equal(back["kexp"][i, i], kx[i])
        assert np.array_equal(back["vexp"][i, i], vx[i])


def test_tq4v2_sizes_and_hand_positions():
    assert layout.tq4v2_record_bytes(128) == 1920 and layout.tq4v2_record_bytes(64) == 928
    sec = layout.tq4v2_sections(128)
    assert (sec["kc"], sec["vc"], sec["vm"], sec["ks"], sec["end"]) == (0, 1024, 1536, 1792, 1824)
    # worked by hand (D = 128, G = 4): channel 0 of token 0 -> byte 0, bit 0;
    # channel 1 -> bit 2; channel 64 (pair 32: gp 2, j 0) -> word 1 -> byte 4;
    # token 5 (r 1, tt 1), channel 35 (pair 17: gp 1, j 1, odd) -> byte
    # ((16 + 1) * 2 + 0) * 4 + 1 = 137, bit 4 + 2 = 6
    assert tuple(map(int, layout.vc2_position(0, 0, 128))) == (0, 0)
    assert tuple(map(int, layout.vc2_position(0, 1, 128))) == (0, 2)
    assert tuple(map(int, layout.vc2_position(0, 64, 128))) == (4, 0)
    assert tuple(map(int, layout.vc2_position(5, 35, 128))) == (137, 6)


@pytest.mark.parametrize("d", [64, 128])
def test_vc2_map_is_a_bijection(d):
    t = np.arange(16)[:, None]
    c = np.arange(d)[None, :]
    pos, shift = layout.vc2_position(t, c, d)
    slots = (pos * 8 + shift).ravel()
    assert len(np.unique(slots)) == 16 * d
    assert pos.min() == 0 and pos.max() == 16 * d // 4 - 1
    assert set(np.unique(shift).tolist()) == {0, 2, 4, 6}


@pytest.mark.parametrize("d", [64, 128])
def test_tq4v2_write_read_round_trip(d):
    rng = np.random.default_rng(41 + d)
    n = 16
    kc = rng.integers(0, 16, size=(n, d)).astype(np.uint8)
    vc = rng.integers(0, 4, size=(n, d)).astype(np.uint8)
    ks = rng.standard_normal(n).astype(np.float16)
    vs = rng.standard_normal((n, d // 32)).astype(np.float16)
    vm = rng.standard_normal((n, d // 32)).astype(np.float16)
    buf = np.zeros(layout.tq4v2_record_bytes(d), np.uint8)
    layout.tq4v2_write_rows(buf, np.zeros(n, np.int64), np.arange(n), d, kc, ks, vc, vs, vm)
    out = layout.tq4v2_read_block(buf[None], d)
    assert np.array_equal(out["kcode"][0], kc) and np.array_equal(out["vcode"][0], vc)
    assert np.array_equal(out["kscale"][0], ks)
    assert np.array_equal(out["vscale"][0], vs) and np.array_equal(out["vmin"][0], vm)
