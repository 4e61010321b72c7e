"""The C ABI from C: include/attn53.h compiles as strict C99 (and as C++17), every function
it declares links against the built library, and the host-only calls behave as documented
when made from a C program (no GPU is touched: the invalid call is rejected before any
launch)."""
import os
import re
import shutil
import subprocess

import pytest

import exact_attention_53_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn53.h")
ROCM_LIB = "/opt/rocm/lib"


def _declared():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", src)))


def _program() -> str:
    refs = "\n".join(f"  (void)&{n};" for n in _declared())
    return f"""#include "attn53.h"
#include <stdio.h>

int main(void) {{
  attn_strides s;
  attn_status st;
{refs}
  s.b = 0;
  s.h = 0;
  s.t = 0;
  /* B = 0: rejected on the host, nothing launched */
  st = attn_fwd(NULL, s, NULL, s, NULL, s, NULL, s, NULL, 0, 1, 1, 64, 64, 0.125f, 1, NULL);
  printf("%d\\n%d\\n%s\\n%lu\\n", attn_version(), (int)st, attn_status_string(st),
         (unsigned long)attn_bwd_workspace_bytes(1, 2, 128, 64, 64, 1));
  return 0;
}}
"""


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++17")])
def test_header_compiles_links_and_runs(tmp_path, compiler, std):
    if not os.path.exists(attn.lib_path):
        pytest.fail("libattn53.so is not built: run __graft_entry__.build()")
    cc = shutil.which(compiler)
    if cc is None:
        pytest.skip(f"{compiler} not available")
    src = tmp_path / ("prog.c" if compiler == "gcc" else "prog.cpp")
    src.write_text(_program())
    exe = tmp_path / "prog"
    libdir = os.path.dirname(attn.lib_path)
    cmd = [cc, std, "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-o", str(exe), f"-L{libdir}", "-l:libattn53.so", f"-Wl,-rpath,{libdir}",
           f"-Wl,-rpath-link,{ROCM_LIB}", f"-Wl,-rpath,{ROCM_LIB}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    version, status, text, ws = out.stdout.splitlines()
    lib = attn.load()
    assert int(version) == lib.attn_version()
    assert int(status) == 2  # ATTN_ERR_SHAPE
    assert text == lib.attn_status_string(2).decode()
    assert int(ws) == lib.attn_bwd_workspace_bytes(1, 2, 128, 64, 64, 1)
