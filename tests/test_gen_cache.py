"""The workload cache: cached_config(i) returns exactly make_config(i), from
disk on the second call, and regenerates a cache whose files no longer match
their manifest (checksums) or whose generator changed (version)."""

import json
import os

import numpy as np

import gen


def same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        if isinstance(a[k], np.ndarray):
            assert a[k].dtype == b[k].dtype and np.array_equal(a[k], b[k]), k
        else:
            assert a[k] == b[k], k


def test_cache_roundtrip_and_corruption(tmp_path):
    ref = gen.make_config(0)
    a = gen.cached_config(0, root=str(tmp_path))
    same(a, ref)
    d = tmp_path / "cfg0"
    man = json.loads((d / "manifest.json").read_text())
    assert man["config"] == "dense-1k-f32" and set(man["arrays"]) >= {"Q", "K", "V", "dO"}
    # second call loads from disk (files untouched)
    mtime = os.path.getmtime(d / "Q.npy")
    b = gen.cached_config(0, root=str(tmp_path))
    same(b, ref)
    assert os.path.getmtime(tmp_path / "cfg0" / "Q.npy") == mtime
    # a flipped byte in one array fails its checksum: the cache is rebuilt
    q = bytearray((d / "Q.npy").read_bytes())
    q[-1] ^= 0xFF
    (d / "Q.npy").write_bytes(bytes(q))
    c = gen.cached_config(0, root=str(tmp_path))
    same(c, ref)
    assert gen._sha256_file(str(tmp_path / "cfg0" / "Q.npy")) == man["arrays"]["Q"]["sha256"]


def test_cache_rebuilt_for_another_generator_version(tmp_path):
    gen.cached_config(0, root=str(tmp_path))
    p = tmp_path / "cfg0" / "manifest.json"
    man = json.loads(p.read_text())
    man["generator_version"] = "0" * 64
    p.write_text(json.dumps(man))
    same(gen.cached_config(0, root=str(tmp_path)), gen.make_config(0))
    assert json.loads(p.read_text())["generator_version"] == gen._generator_version()
