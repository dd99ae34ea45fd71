"""The expert bank's manifest: the fields "Beam 1.0 501B-A23B, streaming pack,
NVFP4 experts / MLX 8-bit residents" ("What this pack holds", routed-experts
and global-scales bullets) lists for expert-manifest.json: the format and
layout names, the 9 parts of a record, each record's offset, length and
SHA-256, and the projections whose global scale is inexact.

Host-side assembly only: the digests come from moe_nvfp4_record_sha256 (a
device kernel over the records as they sit in memory), the inexact flags from
moe_nvfp4_global_from_ws2.
"""
import json

import torch

from . import lib, moe_nvfp4_record_sha256

FORMAT = "mlx-stream-nvfp4-expert-bank-v1"
LAYOUT = "nvfp4-gud-9part"
PROJECTIONS = ("gate", "up", "down")


def part_table(bank):
    """[(name, offset, length)] of a record's 9 parts, in the bank's order."""
    n = bank.H * bank.I
    parts = []
    for p, name in enumerate(PROJECTIONS):
        parts.append((f"{name}.codes", int(bank.part_off[2 * p]), n // 2))
        parts.append((f"{name}.scales", int(bank.part_off[2 * p + 1]), n // 16))
    for p, name in enumerate(PROJECTIONS):
        parts.append((f"{name}.global", int(bank.part_off[6 + p]), 4))
    return sorted(parts, key=lambda t: t[1])


def record_digests(bank, chunk=256, stream=None):
    """SHA-256 of every record (hex strings), computed on the device."""
    out = []
    for e0 in range(0, bank.E, chunk):
        n = min(chunk, bank.E - e0)
        d = torch.empty((n, 32), dtype=torch.uint8, device="cuda")
        moe_nvfp4_record_sha256(bank, e0, n, d, stream)
        out += [bytes(row).hex() for row in d.cpu().numpy()]
    return out


def bank_manifest(bank, inexact=None, source=None, stream=None):
    """The manifest as a dict. inexact: optional [E][3] flags (gate, up, down)
    from moe_nvfp4_global_from_ws2; source: optional provenance string."""
    lib()
    digests = record_digests(bank, stream=stream)
    m = {
        "format": FORMAT,
        "layout": LAYOUT,
        "H": bank.H, "I": bank.I, "experts": bank.E,
        "record_bytes": int(bank.record_bytes), "stride": int(bank.stride),
        "parts": [{"name": n, "offset": o, "length": l} for n, o, l in part_table(bank)],
        "records": [{"offset": e * int(bank.stride), "length": int(bank.record_bytes), "sha256": digests[e]}
                    for e in range(bank.E)],
        "global_scale_inexact": [],
    }
    if source is not None:
        m["source"] = source
    if inexact is not None:
        for e in range(bank.E):
            for p, name in enumerate(PROJECTIONS):
                if inexact[e][p]:
                    m["global_scale_inexact"].append({"record": e, "projection": name})
    return m


def write_manifest(path, bank, inexact=None, source=None):
    with open(path, "w") as f:
        json.dump(bank_manifest(bank, inexact, source), f, indent=1)
