"""A small GGUF writer for tests (versions 2 and 3): header, metadata of every
value type, tensor infos, aligned data.  It writes the published container
layout and holds none of the product's arithmetic."""
from __future__ import annotations

import struct

# metadata value types
U8, I8, U16, I16, U32, I32, F32, BOOL, STRING, ARRAY, U64, I64, F64 = range(13)
_FMT = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f", BOOL: "<?",
        U64: "<Q", I64: "<q", F64: "<d"}


def _string(s: str) -> bytes:
    b = s.encode()
    return struct.pack("<Q", len(b)) + b


def _value(t: int, v) -> bytes:
    if t == STRING:
        return _string(v)
    if t == ARRAY:
        et, items = v
        body = b"".join(_string(x) if et == STRING else struct.pack(_FMT[et], x) for x in items)
        return struct.pack("<IQ", et, len(items)) + body
    return struct.pack(_FMT[t], v)


def write_gguf(path, metadata, tensors, alignment: int = 32, version: int = 3, magic: bytes = b"GGUF"):
    """metadata: [(key, type, value)]; tensors: [(name, type_id, dims innermost first, bytes)].
    Returns the absolute data offset of every tensor, in order."""
    head = bytearray(magic + struct.pack("<IQQ", version, len(tensors), len(metadata)))
    for key, t, v in metadata:
        head += _string(key) + struct.pack("<I", t) + _value(t, v)
    rel, pos = [], 0
    for _, _, _, data in tensors:
        pos = (pos + alignment - 1) // alignment * alignment
        rel.append(pos)
        pos += len(data)
    for (name, tid, dims, _), off in zip(tensors, rel):
        head += _string(name) + struct.pack("<I", len(dims)) + b"".join(struct.pack("<Q", d) for d in dims)
        head += struct.pack("<IQ", tid, off)
    data_start = (len(head) + alignment - 1) // alignment * alignment
    blob = bytearray(head + b"\0" * (data_start - len(head)))
    for (_, _, _, data), off in zip(tensors, rel):
        blob += b"\0" * (data_start + off - len(blob))
        blob += data
    with open(path, "wb") as f:
        f.write(blob)
    return [data_start + o for o in rel]
