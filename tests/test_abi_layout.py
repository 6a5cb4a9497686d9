"""The binding's ctypes structures match the C layouts of include/cqsa.h.

A small C program compiled against the header prints sizeof and offsetof of every
field of the public structs; the ctypes mirrors must agree byte for byte, or the
binding would read and write the wrong fields.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

from memory_bounded_streaming_amd import cqsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRUCTS = {
    "cqsa_plan_info": cqsa.PlanInfo,
    "cqsa_stats": cqsa.Stats,
    "cqsa_rates": cqsa.Rates,
    "cqsa_estimate": cqsa.Estimate,
}


def _c_layout(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "cqsa.h"', "int main(void) {"]
    for cname, ct in STRUCTS.items():
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in ct._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    table = {}
    for line in out.splitlines():
        cname, field, value = line.split()
        table[(cname, field)] = int(value)
    return table


def test_ctypes_structs_match_header(tmp_path):
    table = _c_layout(tmp_path)
    for cname, ct in STRUCTS.items():
        assert ctypes.sizeof(ct) == table[(cname, "sizeof")], cname
        for fname, _ in ct._fields_:
            assert getattr(ct, fname).offset == table[(cname, fname)], f"{cname}.{fname}"


CONSTANTS = ["CQSA_OK", "CQSA_EINVAL", "CQSA_ENOSET", "CQSA_EDIVIDE", "CQSA_EBUDGET", "CQSA_EHIP", "CQSA_ENOMEM",
             "CQSA_ESMALL", "CQSA_BF16", "CQSA_F32", "CQSA_RES_DEVICE", "CQSA_RES_HOST_PINNED",
             "CQSA_FLAG_HOST_ACC", "CQSA_FLAG_KV_SINGLE", "CQSA_FLAG_PAD", "CQSA_FLAG_CAUSAL", "CQSA_FLAG_FREE_BUDGET"]


def test_binding_constants_match_header(tmp_path):
    """Every status, dtype, residency and flag value the binding mirrors equals the header's."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ["#include <stdio.h>", '#include "cqsa.h"', "int main(void) {"]
    lines += [f'  printf("{name} %lld\\n", (long long)({name}));' for name in CONSTANTS]
    lines += ["  return 0;", "}"]
    src = tmp_path / "constants.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "constants"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    header = {name: int(value) for name, value in (line.split() for line in out.splitlines())}
    assert header == {name: getattr(cqsa, name) for name in CONSTANTS}
