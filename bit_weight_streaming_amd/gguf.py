"""Reader for GGUF model files (version 2 and 3): metadata, tensor table and
the raw bytes of each tensor, so that a Q4_K_M file's matrices can go to
`repack` (Q4_K) and `q6k_repack` (Q6_K).

GGUF layout (little-endian throughout):
  uint32 magic "GGUF", uint32 version, uint64 tensor count, uint64 metadata count;
  metadata entries: string key, uint32 value type, value;
  tensor infos: string name, uint32 n_dims, uint64 dims[n_dims] (dims[0] the
  innermost, i.e. the length of a row), uint32 ggml type, uint64 offset into
  the data section;
  the data section, starting at the first multiple of `general.alignment`
  (32 when absent) after the tensor infos.
A string is a uint64 length and that many UTF-8 bytes; an array is a uint32
element type, a uint64 count and the elements.

Host-side only: nothing here touches the GPU.
"""
from __future__ import annotations

import struct
from dataclasses import dataclass

import numpy as np

GGUF_MAGIC = b"GGUF"

# metadata value types
_SCALARS = {0: "<B", 1: "<b", 2: "<H", 3: "<h", 4: "<I", 5: "<i", 6: "<f", 7: "<?",
            10: "<Q", 11: "<q", 12: "<d"}
T_STRING, T_ARRAY = 8, 9

# ggml tensor types this library multiplies, and the plain ones a file holds
# beside them: (name, weights per block, bytes per block)
GGML_TYPES = {0: ("F32", 1, 4), 1: ("F16", 1, 2), 8: ("Q8_0", 32, 34), 12: ("Q4_K", 256, 144),
              14: ("Q6_K", 256, 210)}
Q4_K, Q6_K = 12, 14


class GGUFError(ValueError):
    pass


@dataclass
class TensorInfo:
    name: str
    dims: tuple          # dims[0] innermost (row length)
    type: int            # ggml type id
    offset: int          # absolute byte offset in the file
    nbytes: int          # 0 for types this reader cannot size

    @property
    def type_name(self) -> str:
        return GGML_TYPES.get(self.type, (f"type{self.type}",))[0]

    @property
    def rows(self) -> int:
        n = 1
        for d in self.dims[1:]:
            n *= d
        return n

    @property
    def row_len(self) -> int:
        return self.dims[0] if self.dims else 1


class _Cursor:
    def __init__(self, buf):
        self.buf, self.pos = buf, 0

    def take(self, fmt):
        size = struct.calcsize(fmt)
        if self.pos + size > len(self.buf):
            raise GGUFError("file ends inside the header")
        v = struct.unpack_from(fmt, self.buf, self.pos)[0]
        self.pos += size
        return v

    def string(self):
        n = self.take("<Q")
        if self.pos + n > len(self.buf):
            raise GGUFError("file ends inside a string")
        s = bytes(self.buf[self.pos:self.pos + n]).decode("utf-8")
        self.pos += n
        return s

    def value(self, vtype):
        if vtype in _SCALARS:
            return self.take(_SCALARS[vtype])
        if vtype == T_STRING:
            return self.string()
        if vtype == T_ARRAY:
            etype, count = self.take("<I"), self.take("<Q")
            return [self.value(etype) for _ in range(count)]
        raise GGUFError(f"unknown metadata value type {vtype}")


class GGUF:
    """A GGUF file opened read-only: `metadata` (dict), `tensors` (dict name ->
    TensorInfo), `data_offset`, and `tensor_bytes(name)` (a read-only uint8
    view of the mapped file)."""

    def __init__(self, path: str):
        self.path = path
        self._map = np.memmap(path, dtype=np.uint8, mode="r")
        cur = _Cursor(memoryview(self._map))
        if bytes(self._map[:4]) != GGUF_MAGIC:
            raise GGUFError("not a GGUF file (bad magic)")
        cur.pos = 4
        self.version = cur.take("<I")
        if self.version not in (2, 3):
            raise GGUFError(f"unsupported GGUF version {self.version}")
        n_tensors, n_kv = cur.take("<Q"), cur.take("<Q")
        self.metadata = {}
        for _ in range(n_kv):
            key = cur.string()
            self.metadata[key] = cur.value(cur.take("<I"))
        infos = []
        for _ in range(n_tensors):
            name = cur.string()
            n_dims = cur.take("<I")
            dims = tuple(cur.take("<Q") for _ in range(n_dims))
            infos.append((name, dims, cur.take("<I"), cur.take("<Q")))
        align = int(self.metadata.get("general.alignment", 32))
        if align < 1:
            raise GGUFError("bad general.alignment")
        self.data_offset = (cur.pos + align - 1) // align * align
        self.tensors = {}
        for name, dims, ttype, off in infos:
            nbytes = 0
            if ttype in GGML_TYPES:
                _, per_block, block_bytes = GGML_TYPES[ttype]
                count = int(np.prod(dims, dtype=np.int64)) if dims else 1
                if dims and dims[0] % per_block:
                    raise GGUFError(f"{name}: row length {dims[0]} is not a multiple of {per_block}")
                nbytes = count // per_block * block_bytes
            start = self.data_offset + off
            if start + nbytes > self._map.size:
                raise GGUFError(f"{name}: data runs past the end of the file")
            self.tensors[name] = TensorInfo(name, dims, ttype, start, nbytes)

    def tensor_bytes(self, name: str) -> np.ndarray:
        t = self.tensors[name]
        if t.nbytes == 0:
            raise GGUFError(f"{name}: type {t.type_name} is not one this reader sizes")
        return self._map[t.offset:t.offset + t.nbytes]

    def matrix(self, name: str):
        """(uint8 rows [N, K/256 * block bytes], N, K, ggml type) of a Q4_K or
        Q6_K weight matrix, ready for `repack` / `q6k_repack`."""
        t = self.tensors[name]
        if t.type not in (Q4_K, Q6_K) or len(t.dims) != 2:
            raise GGUFError(f"{name}: a 2-D Q4_K or Q6_K matrix is expected, found "
                            f"{t.type_name} {t.dims}")
        K, N = t.dims
        return self.tensor_bytes(name).reshape(N, -1), N, K, t.type
