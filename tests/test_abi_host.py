"""Host-side checks of the C ABI (CPU only; no device work is enqueued):
the library loads and exports every function include/ddl.h declares, the
Python structures match the C layouts, and the pure host logic (layer
admission, blob sizing, mirror capacity policy and bookkeeping) behaves as
specified."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddl.h")


@pytest.fixture(scope="module")
def ddl():
    import dense_decoder_layer_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddl_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function(ddl):
    from dense_decoder_layer_amd import _native
    names = declared_functions()
    assert len(names) == 26
    lib = _native.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ddl.h but not exported"
        assert n in _native.SIGNATURES, f"{n} has no Python binding"
    out = subprocess.run(["nm", "-D", "--defined-only", _native.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (ddl_\w+)", out))
    assert set(names) <= exported
    assert set(_native.SIGNATURES) == set(names)


def test_struct_layouts_match_c(ddl, tmp_path):
    from dense_decoder_layer_amd import _native as N
    fields = {
        "ddl_ctx_opts": (N.CtxOpts, ["min_batch", "fault_after_admission", "attn_form"]),
        "ddl_layer_desc": (N.LayerDesc, [f for f, _ in N.LayerDesc._fields_]),
        "ddl_layer_weights": (N.LayerWeights, [f for f, _ in N.LayerWeights._fields_]),
    }
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "ddl.h"', "int main(void){"]
    for cname, (_, fs) in fields.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f in fs:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True,
                               check=True).stdout.splitlines():
        c, f, v = line.split()
        got[(c, f)] = int(v)
    for cname, (cls, fs) in fields.items():
        assert ctypes.sizeof(cls) == got[(cname, "sizeof")], cname
        for f in fs:
            assert getattr(cls, f).offset == got[(cname, f)], (cname, f)


def test_mirror_capacity_policy(ddl):
    # planned capacity when it holds rows+1, else max(next_pow2(rows+1), 512)
    assert ddl.ddl_mirror_plan_capacity(0) == 512
    assert ddl.ddl_mirror_plan_capacity(32) == 512
    assert ddl.ddl_mirror_plan_capacity(300) == 512
    assert ddl.ddl_mirror_plan_capacity(511) == 512
    assert ddl.ddl_mirror_plan_capacity(512) == 1024
    assert ddl.ddl_mirror_plan_capacity(4096) == 8192
    assert ddl.ddl_mirror_plan_capacity(32768) == 65536
    assert ddl.ddl_mirror_plan_capacity(100, 4096) == 4096
    assert ddl.ddl_mirror_plan_capacity(4096, 4096) == 8192     # planned < rows + 1
    assert ddl.ddl_mirror_plan_capacity(4095, 4096) == 4096
    assert ddl.ddl_mirror_plan_capacity(-1) < 0


def test_mirror_bookkeeping_without_device_work(ddl):
    from dense_decoder_layer_amd import _native as N
    lib = N.lib()
    assert ddl.ddl_mirror_bytes(8, 128, 512) == 2 * 512 * 8 * 128 * 4
    assert ddl.ddl_mirror_bytes(0, 128, 512) == 0
    fake = ctypes.c_void_p(0x1000)     # never dereferenced by these calls
    m = ctypes.c_void_p()
    assert lib.ddl_mirror_init(ctypes.byref(m), fake, 100, 8, 128, 512) == ddl.DDL_ERR_INVALID
    assert lib.ddl_mirror_init(ctypes.byref(m), fake, 1 << 30, 8, 128, 512) == 1
    assert lib.ddl_mirror_seq_len(m) == 0 and lib.ddl_mirror_capacity(m) == 512
    # more rows than the capacity: error, no copy enqueued, the mirror goes stale
    assert lib.ddl_mirror_upload(m, fake, fake, 513, None) == ddl.DDL_ERR_INVALID
    assert lib.ddl_mirror_seq_len(m) == -1
    lib.ddl_mirror_invalidate(m)
    assert lib.ddl_mirror_seq_len(m) == -1
    lib.ddl_mirror_destroy(m)


def test_layer_admission_predicates(ddl):
    ok = dict(d_model=3072, n_heads=24, n_kv_heads=8, head_dim=128, d_ff=8192)
    assert ddl.ddl_layer_supported(ddl.layer_desc(**ok))
    assert ddl.ddl_layer_blob_bytes(ddl.layer_desc(**ok)) >= 2 * 100663296
    refusals = [
        (dict(act=7), "activation"),
        (dict(post_norm_eps=1e-6), "epsilon"),
        (dict(v_head_dim=64), "v_head_dim"),
        (dict(window=-1), "window"),
        (dict(has_sinks=1), "sinks"),
        (dict(has_alibi=1), "ALiBi"),
        (dict(has_lora=1), "LoRA"),
        (dict(rope_layout=5), "layout"),
        (dict(rope_rot_dim=96), "multiple of 64"),          # Neox pairs e, e+48
        (dict(rope_rot_dim=130, rope_layout=ddl.DDL_ROPE_NORM), "head_dim"),
        (dict(rope_rot_dim=63, rope_layout=ddl.DDL_ROPE_NORM), "even"),
        (dict(rope_mscale=float("inf")), "factor"),
        (dict(rope_freq_factors=[1.0] * 63 + [0.0]), "frequency factor"),
    ]
    for extra, why in refusals:
        d = ddl.layer_desc(**ok, **extra)
        assert not ddl.ddl_layer_supported(d), extra
        assert why in ddl.ddl_last_error(), (extra, ddl.ddl_last_error())
        assert ddl.ddl_layer_blob_bytes(d) == 0
    assert not ddl.ddl_layer_supported(ddl.layer_desc(3072, 24, 8, 96, 8192))
    assert not ddl.ddl_layer_supported(ddl.layer_desc(3072, 24, 7, 128, 8192))
    assert not ddl.ddl_layer_supported(ddl.layer_desc(3000, 24, 8, 128, 8192))
    # a layer without RoPE is served, and so are the RoPE, activation and
    # window options the kernels implement
    assert ddl.ddl_layer_supported(ddl.layer_desc(**ok, rope_theta=None))
    served = [dict(act=ddl.DDL_ACT_GELU), dict(window=4096), dict(rope_layout=ddl.DDL_ROPE_NORM),
              dict(rope_layout=ddl.DDL_ROPE_NORM, rope_rot_dim=96), dict(rope_rot_dim=64),
              dict(rope_mscale=0.5), dict(rope_freq_factors=[1.0 + i / 8 for i in range(64)]),
              dict(has_post_attn_norm=1), dict(has_post_ffn_norm=1),
              dict(has_post_attn_norm=1, has_post_ffn_norm=1)]
    for extra in served:
        assert ddl.ddl_layer_supported(ddl.layer_desc(**ok, **extra)), (extra, ddl.ddl_last_error())


def test_blob_bytes_cover_the_packed_matrices(ddl):
    d = ddl.layer_desc(4096, 32, 8, 128, 14336, qkv_bias=True, qk_norm=True)
    params = (4096 + 2 * 1024) * 4096 + 4096 * 4096 + 3 * 14336 * 4096
    assert 2 * params < ddl.ddl_layer_blob_bytes(d) < 2 * params + 65536
    g = ddl.layer_desc(4096, 32, 8, 128, 14336, gated=True)
    assert ddl.ddl_layer_blob_bytes(g) - ddl.ddl_layer_blob_bytes(
        ddl.layer_desc(4096, 32, 8, 128, 14336)) == 2 * 4096 * 4096


def test_context_create_destroy_touches_no_device(ddl):
    c = ddl.ddl_ctx_create(min_batch=1)
    ddl.ddl_ctx_destroy(c)
    assert c.handle is None


def test_oracle_and_gpu_path_share_no_code():
    import_re = re.compile(r"^\s*(?:from|import)\s+([\w.]+)", re.M)
    pkg = os.path.join(ROOT, "dense_decoder_layer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                mods = import_re.findall(open(os.path.join(dirpath, f)).read())
                assert not any(m.split(".")[0] in ("oracle", "synth", "tests") for m in mods), f
            if f.endswith((".hip", ".cpp", ".h")):
                assert "oracle" not in open(os.path.join(dirpath, f)).read(), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            mods = import_re.findall(open(os.path.join(ROOT, "oracle", f)).read())
            assert not any(m.split(".")[0] in ("dense_decoder_layer_amd", "synth") for m in mods)
    for f in os.listdir(os.path.join(ROOT, "synth")):
        if f.endswith(".py"):
            mods = import_re.findall(open(os.path.join(ROOT, "synth", f)).read())
            assert not any(m.split(".")[0] in ("dense_decoder_layer_amd", "oracle") for m in mods)


def test_build_works_in_a_checkout_without_the_library(tmp_path):
    # __graft_entry__.build() must build before it imports the package (which
    # refuses to load without the library).  In a copy of the tree without
    # libddl.so, a stand-in build script places the library built here
    # (compiling again would take minutes).
    import shutil
    import sys as _sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib = os.path.join(root, "dense_decoder_layer_amd", "libddl.so")
    shutil.copy(os.path.join(root, "__graft_entry__.py"), tmp_path)
    shutil.copytree(os.path.join(root, "dense_decoder_layer_amd"), tmp_path / "dense_decoder_layer_amd",
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__", "csrc"))
    assert not (tmp_path / "dense_decoder_layer_amd" / "libddl.so").exists()
    (tmp_path / "dense_decoder_layer_amd" / "build.py").write_text(
        "import os, shutil\n"
        "def build(verbose=False):\n"
        f"    shutil.copy({lib!r}, os.path.join(os.path.dirname(os.path.abspath(__file__)), 'libddl.so'))\n")
    r = subprocess.run([_sys.executable, "-c", "import __graft_entry__ as g; g.build()"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert (tmp_path / "dense_decoder_layer_amd" / "libddl.so").exists()


def test_empty_and_short_batches_decline_before_touching_anything(ddl):
    """A call with no new tokens (or fewer than the context's min_batch) is
    declined before any pointer is read: the pointers here are host
    sentinels that a device access would fault on, and the layer pointer
    is never dereferenced."""
    from dense_decoder_layer_amd import _native as N
    lib = N.lib()
    ctx = ddl.ddl_ctx_create(min_batch=4)
    sentinel = ctypes.c_void_p(0x1000)
    layers = (ctypes.c_void_p * 1)(0x2000)
    rows_arr = (ctypes.c_void_p * 1)(0x3000)
    prefix_rows = (ctypes.c_int * 1)(0)
    for batch in (0, 3):
        rc = lib.ddl_prefill_dense_stack(ctx.handle, sentinel, layers, 1, batch, 0, None, None,
                                         prefix_rows, sentinel, rows_arr, rows_arr, sentinel,
                                         0, None)
        assert rc == ddl.DDL_DECLINED, (batch, rc)
        assert b"min_batch" in lib.ddl_last_error()
    ddl.ddl_ctx_destroy(ctx)
