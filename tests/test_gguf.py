"""The GGUF reader on files written here by the format's definition (no real
model file exists in this environment): metadata of every kind, tensors of
the types the library multiplies, alignment of the data section, errors."""
import struct

import numpy as np
import pytest

import oracle
import synth
from bit_weight_streaming_amd import gguf


def _s(text):
    b = text.encode()
    return struct.pack("<Q", len(b)) + b


def _write(path, kvs, tensors, align=32):
    """kvs: [(key, type id, packed value bytes)]; tensors: [(name, dims, type, bytes)]."""
    head = b"GGUF" + struct.pack("<IQQ", 3, len(tensors), len(kvs))
    for key, vtype, payload in kvs:
        head += _s(key) + struct.pack("<I", vtype) + payload
    offs, off = [], 0
    for _, _, _, data in tensors:
        offs.append(off)
        off += (len(data) + align - 1) // align * align
    for (name, dims, ttype, _), o in zip(tensors, offs):
        head += _s(name) + struct.pack("<I", len(dims)) + b"".join(struct.pack("<Q", d) for d in dims)
        head += struct.pack("<IQ", ttype, o)
    head += b"\0" * ((-len(head)) % align)
    body = b""
    for (_, _, _, data), o in zip(tensors, offs):
        body += b"\0" * (o - len(body)) + data
    with open(path, "wb") as f:
        f.write(head + body)


def test_reads_metadata_and_tensors(tmp_path):
    q6 = synth.q6k_matrix(synth.key(1, 14, 3, 512), 3, 512)
    q4 = synth.q4k_matrix(synth.key(1, 12, 2, 256), 2, 256)
    f16 = np.arange(32, dtype=np.float16)
    kvs = [("general.architecture", 8, _s("test")),
           ("general.alignment", 4, struct.pack("<I", 64)),
           ("test.layers", 9, struct.pack("<IQ", 5, 3) + struct.pack("<3i", 1, -2, 3)),
           ("test.eps", 6, struct.pack("<f", 1e-6)),
           ("test.flag", 7, struct.pack("<?", True)),
           ("test.big", 10, struct.pack("<Q", 2 ** 40))]
    tensors = [("blk.0.ffn_down.weight", (512, 3), 14, q6.tobytes()),
               ("blk.0.attn_q.weight", (256, 2), 12, q4.tobytes()),
               ("token_embd.weight", (8, 4), 1, f16.tobytes())]
    path = tmp_path / "t.gguf"
    _write(path, kvs, tensors, align=64)
    g = gguf.GGUF(str(path))
    assert g.version == 3
    assert g.metadata["general.architecture"] == "test"
    assert g.metadata["test.layers"] == [1, -2, 3]
    assert abs(g.metadata["test.eps"] - 1e-6) < 1e-12 and g.metadata["test.flag"] is True
    assert g.metadata["test.big"] == 2 ** 40
    assert g.data_offset % 64 == 0
    W, N, K, t = g.matrix("blk.0.ffn_down.weight")
    assert (N, K, t) == (3, 512, gguf.Q6_K) and np.array_equal(W, q6)
    assert np.array_equal(oracle.q6k_dequant_rows(W, 512), oracle.q6k_dequant_rows(q6, 512))
    W, N, K, t = g.matrix("blk.0.attn_q.weight")
    assert (N, K, t) == (2, 256, gguf.Q4_K) and np.array_equal(W, q4)
    e = g.tensors["token_embd.weight"]
    assert e.type_name == "F16" and e.rows == 4 and e.row_len == 8
    assert np.array_equal(g.tensor_bytes("token_embd.weight").view(np.float16), f16)
    with pytest.raises(gguf.GGUFError):
        g.matrix("token_embd.weight")


def test_rejects_bad_files(tmp_path):
    p = tmp_path / "bad.gguf"
    p.write_bytes(b"GGML" + b"\0" * 60)
    with pytest.raises(gguf.GGUFError):
        gguf.GGUF(str(p))
    q6 = synth.q6k_matrix(synth.key(2, 14, 1, 256), 1, 256)
    _write(p, [], [("w", (256, 1), 14, q6.tobytes())])
    data = p.read_bytes()
    p.write_bytes(data[:-10])               # data cut short
    with pytest.raises(gguf.GGUFError):
        gguf.GGUF(str(p))
