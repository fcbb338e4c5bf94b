"""The C-ABI library loads on a CPU-only host, exports every function include/ec.h
declares, and rejects bad arguments on the host with the documented status
codes (no call here reaches a kernel launch)."""
import ctypes as C
import os
import re

import pytest

from entropy_gated_kv_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ec.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(ec_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


def test_version_and_status_strings(lib):
    assert lib.ec_abi_version() == 6
    for s in range(-7, 1):
        assert lib.ec_status_string(s)
    assert lib.ec_status_string(99) == b"unknown status"


def test_workspace_queries(lib):
    assert lib.ec_entropy_workspace_bytes(4096, 126464) >= 4096 * 8 * 16
    assert lib.ec_entropy_workspace_bytes(0, 10) == 0
    assert lib.ec_attention_workspace_bytes(0, 1, 1, 1, 32) == 0


def test_step_workspace_grows_with_the_block_bound(lib):
    """A workspace sized for a block bound serves every shorter block, also
    without a logits buffer, where a packed LM head's statistics need one
    16-byte partial per row (up to 32) and group of column tiles."""
    layers = (L.ec_layer * 1)(L.ec_layer(FAKE, FAKE, None, None, None, None, None))
    m = L.ec_model(n_layers=1, d=256, Hq=2, Hkv=2, dh=128, d_ffn=0, V=40032, L_cap=256, dtype=1,
                   rms_eps=1e-5, tok_emb=FAKE, pos_emb=FAKE, layers=layers, norm_final=None, w_lm=FAKE,
                   logit_scale=None, w_lm_packed=FAKE)
    sizes = [lib.ec_step_workspace_bytes(C.byref(m), b) for b in (1, 8, 16, 32, 33, 64, 256)]
    assert all(x > 0 for x in sizes) and sizes == sorted(sizes), sizes
    assert sizes[3] >= 32 * ((40032 + 63) // 64) * 16          # 32 rows x 626 groups


FAKE = 1 << 20       # an aligned, never dereferenced address
ODD = FAKE + 4       # misaligned


def test_entropy_argument_checks(lib):
    f = lib.ec_entropy_max
    ws = lib.ec_entropy_workspace_bytes(4, 100)
    args = [FAKE, 1, 4, 100, 104, None, None, 0, 1.0, FAKE, None, None, FAKE, FAKE, FAKE, ws, None]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=None) == -1
    assert call(a1=7) == -3
    assert call(a2=0) == -2
    assert call(a4=99) == -2                 # stride < V
    assert call(a0=ODD) == -5
    assert call(a4=101) == -5                # stride not a multiple of 16 bytes
    assert call(a15=ws - 1) == -4
    assert call(a5=FAKE, a6=None) == -1      # decoded rows without a count


def test_noalloc_entropy_argument_checks(lib):
    """The workspace-free entropy pass refuses, on the host, a call whose
    partial statistics exceed its static array (before any HIP call)."""
    f = lib.ec_entropy_max_noalloc
    base = [FAKE, 1, 4, 100, 104, None, None, 0, 1.0, FAKE, None, None, FAKE, FAKE, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=None) == -1
    assert call(a1=7) == -3
    assert call(a4=99) == -2
    assert call(a0=ODD) == -5
    rows = L.EC_NOALLOC_SCRATCH_BYTES // 16 + 1          # one 16-byte partial per row
    assert call(a2=rows, a3=16, a4=16) == -4
    # V = 4096: one segment per row in bf16, two in fp32
    half = L.EC_NOALLOC_SCRATCH_BYTES // 32 + 1
    assert call(a1=0, a2=half, a3=4096, a4=4096) == -4
    # within the array the host checks pass (without a GPU the device lookup then fails)
    assert call(a1=1, a2=half, a3=4096, a4=4096) not in (-1, -2, -3, -4, -5)
    assert call(a2=rows - 1, a3=16, a4=16) not in (-1, -2, -3, -4, -5)


def test_select_and_refresh_and_attention_checks(lib):
    assert lib.ec_select_rows(FAKE, FAKE, 10, 8, 4, 0, FAKE, FAKE, 16, 4, FAKE, FAKE, None) == -2
    assert lib.ec_select_rows(FAKE, FAKE, 10, 0, 4, 0, FAKE, FAKE, 2, 4, FAKE, FAKE, None) == -2
    assert lib.ec_select_rows(None, FAKE, 10, 0, 4, 0, FAKE, FAKE, 16, 4, FAKE, FAKE, None) == -1
    # block diffusion: the flag is 0 or 1 and needs an explicit block
    assert lib.ec_select_rows(FAKE, FAKE, 10, 0, 4, 2, FAKE, FAKE, 16, 4, FAKE, FAKE, None) == -2
    assert lib.ec_select_rows(FAKE, FAKE, 10, -1, 4, 1, FAKE, FAKE, 16, 4, FAKE, FAKE, None) == -2
    assert lib.ec_kv_refresh(FAKE, 256, FAKE, FAKE, 4, FAKE, 256, 4, 4, 48, 1, FAKE, FAKE, FAKE,
                             16, None, 0, None) == -7              # head dim 48
    assert lib.ec_kv_refresh(FAKE, 64, FAKE, FAKE, 4, FAKE, 64, 4, 4, 32, 1, FAKE, FAKE, FAKE,
                             16, None, 0, None) == -7              # bf16 needs d % 128 == 0
    assert lib.ec_kv_refresh(FAKE, 128, FAKE, FAKE, 4, FAKE, 128, 4, 3, 32, 1, FAKE, FAKE, FAKE,
                             16, None, 0, None) == -2              # Hq % Hkv
    assert lib.ec_kv_refresh(FAKE, 128, FAKE, FAKE, 4, FAKE, 128, 4, 4, 32, 2, FAKE, FAKE, FAKE,
                             16, None, 0, None) == -3
    need = lib.ec_kv_refresh_workspace_bytes(96, 4096, 32, 32, 128, 1)
    assert need > 0
    assert lib.ec_kv_refresh(FAKE, 4096, FAKE, FAKE, 96, FAKE, 4096, 32, 32, 128, 1, FAKE, FAKE,
                             FAKE, 1024, FAKE, need - 1, None) == -4
    assert lib.ec_bidir_attention(FAKE, FAKE, 4, FAKE, FAKE, 17, 16, 4, 4, 32, 0.17, 1, FAKE, FAKE,
                                  1 << 20, None) == -2             # L > L_cap
    assert lib.ec_bidir_attention(FAKE, FAKE, 4, FAKE, FAKE, 8, 16, 4, 4, 32, -1.0, 1, FAKE, FAKE,
                                  1 << 20, None) == -2             # bad scale


def test_step_argument_checks(lib):
    m = L.ec_model()
    assert lib.ec_step_workspace_bytes(C.byref(m), 32) == 0        # n_layers = 0
    st, cfg = L.ec_state(), L.ec_step_cfg()
    assert lib.ec_step(C.byref(m), C.byref(st), C.byref(cfg), FAKE, 0, None, None) == -2
    assert lib.ec_step(None, C.byref(st), C.byref(cfg), FAKE, 0, None, None) == -1


def test_step_rejects_misaligned_weights(lib):
    """Every weight and gain is read in 16-byte vectors: a misaligned one is
    EC_E_ALIGN (checked on the host; the workspace check comes after)."""
    def call(**bad):
        ly = L.ec_layer(**{f: bad.get(f, FAKE) for f in ("w_qkv", "w_o", "norm_attn", "norm_ffn",
                                                          "w_gate", "w_up", "w_down")})
        layers = (L.ec_layer * 1)(ly)
        m = L.ec_model(n_layers=1, d=256, Hq=4, Hkv=4, dh=64, d_ffn=512, V=bad.get("V", 1024), L_cap=256,
                       dtype=bad.get("dtype", 1), rms_eps=1e-5, tok_emb=FAKE, pos_emb=FAKE, layers=layers,
                       norm_final=bad.get("norm_final", FAKE), w_lm=bad.get("w_lm", FAKE), logit_scale=None,
                       w_lm_packed=bad.get("w_lm_packed"))
        caches = (C.c_void_p * 1)(FAKE)
        st = L.ec_state(L=256, tokens=FAKE, is_masked=FAKE, history=FAKE, history_len=FAKE,
                        history_cap=64, full_flag=FAKE, k_cache=caches, v_cache=caches, rows=FAKE,
                        n_rows=FAKE, logits=bad.get("logits", FAKE), row_entropy=FAKE, row_argmax=FAKE, row_top1=FAKE,
                        chosen=FAKE, n_chosen=FAKE, e_max=FAKE, kv_drift=None,
                        attn_out=bad.get("attn_out"))
        cfg = L.ec_step_cfg(tau=1.0, k=16, n_unmask=2, block_start=192, block_len=bad.get("block_len", 32),
                            mode=bad.get("mode", 0))
        return lib.ec_step(C.byref(m), C.byref(st), C.byref(cfg), FAKE, 0, None, None)

    assert call() == -4                                            # only the workspace is short
    for mode in (1, 2):
        assert call(mode=mode) == -4
    assert call(mode=3) == -2                                      # not an EC_MODE_*
    for f in ("w_qkv", "w_o", "norm_attn", "norm_ffn", "w_gate", "w_up", "w_down", "norm_final",
              "attn_out"):
        assert call(**{f: ODD}) == -5, f
    assert call(attn_out=FAKE) == -4                               # aligned: accepted
    # the packed LM head: bf16, V % 16 == 0, aligned, and only with an LM head
    assert call(w_lm_packed=FAKE) == -4
    assert call(w_lm_packed=ODD) == -5
    assert call(w_lm_packed=FAKE, V=1040) == -7                    # V % 32 != 0: no LM head GEMM for it
    assert call(V=1040) == -7
    assert call(V=1040, w_lm=None) == -4                           # no LM head: any V
    assert call(w_lm_packed=FAKE, dtype=0) == -3
    assert call(w_lm_packed=FAKE, w_lm=None) == -1
    # no logits buffer: only where the packed LM head runs (it then writes
    # softmax statistics instead): a packed copy, block <= 32, V > 32704, d % 256 == 0
    assert call(logits=None, w_lm_packed=FAKE, V=32768) == -4      # accepted: the workspace is short
    assert call(logits=None, V=32768) == -1                        # no packed copy
    assert call(logits=None, w_lm=None, V=32768) == -1             # no LM head: the caller's logits are input
    assert call(logits=None, w_lm_packed=FAKE, V=32704) == -7      # 511 column tiles
    assert call(logits=None, w_lm_packed=FAKE, V=32768, block_len=64) == -7
    assert call(logits=ODD, w_lm_packed=FAKE, V=32768) == -5       # a buffer must be aligned


def test_pack_lm_head_argument_checks(lib):
    f = lib.ec_pack_lm_head
    other = FAKE + (1 << 30)
    assert f(None, 1024, 256, 1, other, None) == -1
    assert f(FAKE, 1024, 256, 0, other, None) == -3              # bf16 only
    assert f(FAKE, 1032, 256, 1, other, None) == -2              # V % 16
    assert f(FAKE, 1024, 250, 1, other, None) == -2              # d % 32
    assert f(FAKE, 8, 256, 1, other, None) == -2
    assert f(FAKE, 1024, 256, 1, ODD, None) == -5
    assert f(FAKE, 1024, 256, 1, FAKE + 4096, None) == -2        # overlaps its source


def test_validation_checks_under_host_sanitizers(tmp_path):
    """The entry points' argument checks live in a HIP-free translation unit
    (ec_validate.cpp).  Built with the host compiler's address and
    undefined-behaviour sanitizers, a driver (tests/validate_driver.cpp)
    checks hand-made cases and calls every check with 200000 rounds of seeded
    random arguments, extreme integers included; any sanitizer report aborts
    it."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "validate_driver")
    csrc = os.path.join(ROOT, "entropy_gated_kv_amd", "csrc")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           "-I", csrc, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
           os.path.join(csrc, "ec_validate.cpp"), os.path.join(ROOT, "tests", "validate_driver.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "all expectations held" in r.stdout


def test_plain_cpp_driver_builds_against_the_header(tmp_path):
    """tests/c_abi_driver.cpp, the suite's user of libec.so without the Python
    binding, compiles and links with the host compiler from include/ec.h and
    the HIP runtime alone (the GPU test runs it)."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    lib_dir = os.path.join(ROOT, "entropy_gated_kv_amd")
    if not os.path.exists(os.path.join(lib_dir, "libec.so")):
        pytest.skip("libec.so is not built")
    exe = str(tmp_path / "c_abi_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I",
           os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_abi_driver.cpp"), "-o", exe, "-L", lib_dir, "-lec",
           "-L", "/opt/rocm/lib", "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
