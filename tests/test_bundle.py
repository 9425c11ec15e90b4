"""CPU tests of the model bundle (uw_bundle_*): write, open, read back; the blobs read out of
a bundle still decode to the original weights with the oracle; corruption is reported."""
import numpy as np
import pytest

import decode_gemm_amd as uw
import oracle
import synth


def setup_module():
    oracle.build(force=False)


def _mats():
    rng = np.random.default_rng(5)
    ws = [synth.gen_weight(synth.CONFIGS["tiny"], "w"),
          synth.f32_to_bf16_bits(rng.standard_normal((96, 320), dtype=np.float32) * 0.03),
          np.full((4, 64), 0x3C01, np.uint16)]
    return ws, [uw.encode(w, chunk=c) for w, c in zip(ws, (256, 64, 128))]


def _plans():
    return [{"N": 512, "K": 256, "M": 1, "pipeline": uw.PIPE_DIRECT, "split_k": 1, "t_ms": 0.0123,
             "variant": "skinny rt4 u2 w4"},
            {"N": 96, "K": 320, "M": 1024, "pipeline": uw.PIPE_EXPAND, "split_k": 4, "t_ms": 1.5,
             "variant": uw.variant_by_name("wide 256x256")},
            {"N": 512, "K": 256, "M": 64, "pipeline": uw.PIPE_TRANSCODE, "split_k": 0, "t_ms": 0.5, "variant": -1},
            {"N": 4, "K": 64, "M": 16, "pipeline": uw.PIPE_FULL, "split_k": 0, "t_ms": 0.0, "variant": "no such kernel"}]


def test_round_trip_items_and_plans():
    ws, blobs = _mats()
    names = ["layer0.mlp.gate", "layer0.mlp.down", "single symbol"]
    buf = uw.bundle_write(list(zip(names, blobs)), _plans())
    info = uw.bundle_open(buf, verify=True)
    assert (info.n_items, info.n_plans, info.total_bytes) == (3, 4, buf.size)
    assert buf.size % 256 == 0 and bytes(buf[:4]) == b"UWB1"
    items = uw.bundle_items(buf)
    assert [i[0] for i in items] == names
    for (name, off, nbytes, h), w, b in zip(items, ws, blobs):
        assert off % 256 == 0 and nbytes == b.size and (buf[off: off + nbytes] == b).all()
        assert bytes(h) == b[:256].tobytes()
        # the blob read back out of the bundle decodes, with the oracle, to the weights
        assert (oracle.decode(buf[off: off + nbytes], want=("w",))["w"] == w).all()
    plans = uw.bundle_plans(buf)
    for got, want in zip(plans, _plans()):
        for k in ("N", "K", "M", "pipeline", "split_k"):
            assert got[k] == want[k], k
        assert abs(got["t_ms"] - want["t_ms"]) < 1e-6
    assert plans[0]["variant"] == uw.variant_by_name("skinny rt4 u2 w4") >= 0
    assert plans[1]["variant_name"] == "wide 256x256"
    assert plans[2]["variant"] == -1 and plans[2]["variant_name"] == ""
    assert plans[3]["variant"] == -1 and plans[3]["variant_name"] == "no such kernel"


def test_empty_bundle_and_size_query():
    buf = uw.bundle_write([], [])
    info = uw.bundle_open(buf)
    assert (info.n_items, info.n_plans) == (0, 0) and buf.size == 256


def test_write_rejects_bad_items_and_plans():
    _, blobs = _mats()
    for items, plans in (
            ([("a", blobs[0]), ("a", blobs[1])], []),                 # repeated name
            ([("", blobs[0])], []),                                    # empty name
            ([("x" * 64, blobs[0])], []),                              # name too long
            ([("a", blobs[0])], [dict(_plans()[0], K=100)]),           # K not a multiple of 64
            ([("a", blobs[0])], [dict(_plans()[0], pipeline=9)]),      # no such pipeline
            ([("a", blobs[0])], [dict(_plans()[0], split_k=5)]),       # more slices than groups
    ):
        with pytest.raises(uw.UwError) as e:
            uw.bundle_write(items, plans)
        assert e.value.status == uw.EINVAL
    bad = blobs[0].copy()
    bad[:4] = 0
    with pytest.raises(uw.UwError) as e:
        uw.bundle_write([("a", bad)])
    assert e.value.status == uw.EFORMAT


def test_open_reports_corruption():
    _, blobs = _mats()
    buf = uw.bundle_write([("g", blobs[0]), ("d", blobs[1])], _plans())
    items = uw.bundle_items(buf)
    cases = []
    b = buf.copy()
    b[0] ^= 1
    cases.append(("magic", b, True))
    cases.append(("truncated", buf[: buf.size - 256].copy(), False))
    b = buf.copy()
    b[256 + 5] ^= 0x20  # a byte of the first item's name: the table checksum
    cases.append(("table", b, False))
    b = buf.copy()
    off = items[1][1]
    b[off + items[1][2] // 2] ^= 0x40  # a byte inside the second blob's body
    cases.append(("blob body", b, True))
    for what, bb, verify in cases:
        with pytest.raises(uw.UwError) as e:
            uw.bundle_open(bb, verify=verify)
        assert e.value.status == uw.EFORMAT, what
    # without verify the damaged blob body is not looked at (its header is intact)
    uw.bundle_open(cases[-1][1], verify=False)
