"""The C-ABI library loads and exports every entry point include/*.h declares;
the ctypes structures match the C layout (checked with gcc).  CPU only: no
compute call is made here."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(spec_verify_\w+)\s*\(", text, flags=re.M))
    return names


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("spec_verify_create", "spec_verify_run", "spec_verify_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    from lossless_rejection_sampling_sampler_amd import EXPORTS, load_library
    lib = load_library()
    names = _declared()
    assert names == set(EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (spec_verify_\w+)", out))
    assert names <= exported


def test_status_strings():
    from lossless_rejection_sampling_sampler_amd import status_string
    assert status_string(0) == "ok"
    assert status_string(1) == "invalid argument"
    assert status_string(99) == "unknown status"


def test_ctypes_layout_matches_c(tmp_path):
    from lossless_rejection_sampling_sampler_amd import SVArgs, SVConfig
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stddef.h>
#include <stdio.h>
#include "spec_verify.h"
#define F(T, m) printf(#T "." #m " %zu\\n", offsetof(T, m));
int main(void) {
  printf("sv_config %zu\\n", sizeof(sv_config));
  printf("sv_args %zu\\n", sizeof(sv_args));
  F(sv_config, flags) F(sv_args, draft_offsets) F(sv_args, target_logits) F(sv_args, uniforms)
  F(sv_args, out_tokens) F(sv_args, diag_ratio)
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    lines = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                     check=True).stdout.splitlines())
    assert int(lines["sv_config"]) == ctypes.sizeof(SVConfig)
    assert int(lines["sv_args"]) == ctypes.sizeof(SVArgs)
    assert int(lines["sv_config.flags"]) == SVConfig.flags.offset
    for m in ("draft_offsets", "target_logits", "uniforms", "out_tokens", "diag_ratio"):
        assert int(lines[f"sv_args.{m}"]) == getattr(SVArgs, m).offset, m


def test_create_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    from lossless_rejection_sampling_sampler_amd import SpecVerify, SpecVerifyError
    with pytest.raises(SpecVerifyError):
        SpecVerify(4, 4, 1000, "bf16")
