"""The C ABI's argument validation under AddressSanitizer, on the CPU.

tests/asan/build_host_asan.py (run by build()) compiles the ABI layer
(exact_attention_74_amd/csrc/api.hip) for the host with AddressSanitizer and
links it with stub launchers that launch nothing and report "no device".  A
child process, with the sanitizer runtime preloaded, drives every entry point
through shape, value, NULL, alignment and aliasing errors and through valid
arguments (which reach a stub and return EXATTN_ERR_HIP); any out-of-bounds
or use-after-free access in the validation code aborts the child.
"""
import os
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "asan", "libexattn_host_asan.so")

CHILD = textwrap.dedent(r'''
    import ctypes, sys
    sys.path.insert(0, ROOT)
    import exact_attention_74_amd as ea   # argument types only; the HIP library is not loaded
    lib = ctypes.CDLL(LIB)
    for name, args in ea.SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ea.RESTYPES.get(name, ctypes.c_int)
    OK, NULL, SHAPE, ALIGN, VALUE, HIP, SCRATCH = 0, -1, -2, -3, -4, -5, -6
    P, G = 1 << 20, 1 << 31
    checks = 0
    def expect(got, want, what):
        global checks
        checks += 1
        if got != want:
            print(f"FAIL {what}: {got} != {want}", flush=True)
            sys.exit(3)
    # forwards (B1 H2 N256 d64): valid -> stub, then each error class
    for fn, nptr in ((lib.attn_fwd_bf16, 5), (lib.attn_fwd_bf16_same_phase, 5), (lib.attn_fwd_fp8, 8)):
        ptrs = [P + i * G for i in range(nptr)]
        call = lambda p=ptrs, B=1, H=2, N=256, d=64, c=0, s=0.125: fn(*p, B, H, N, d, c, s, None)
        expect(call(), HIP, "valid forward")
        expect(call(p=[None] + ptrs[1:]), NULL, "NULL q")
        expect(call(d=96), SHAPE, "d=96")
        expect(call(N=-1), SHAPE, "N<0")
        expect(call(s=0.0), VALUE, "scale 0")
        expect(call(c=2), VALUE, "causal 2")
        expect(call(p=[P + 8] + ptrs[1:]), ALIGN, "misaligned q")
        expect(call(p=ptrs[:-2] + [P, ptrs[-1]]), VALUE, "o aliases q")
        expect(call(p=ptrs[:-1] + [ptrs[-2] + 64]), VALUE, "lse inside o")
        expect(call(B=0, p=[None] * nptr), OK, "empty")
        expect(call(p=ptrs[:-1] + [None]), HIP, "lse NULL is allowed")
    # grouped-query forwards
    g = [P + i * G for i in range(5)]
    expect(lib.attn_fwd_bf16_gqa(*g, 1, 8, 2, 256, 128, 1, 0.1, None), HIP, "gqa valid")
    expect(lib.attn_fwd_bf16_gqa(*g, 1, 8, 3, 256, 128, 1, 0.1, None), SHAPE, "gqa 8/3")
    g8 = [P + i * G for i in range(8)]
    expect(lib.attn_fwd_fp8_gqa(*g8, 1, 8, 2, 300, 256, 0, 0.1, None), HIP, "fp8 gqa d256")
    expect(lib.attn_fwd_fp8_gqa(*g8[:3], g8[6] + 4, *g8[4:], 1, 8, 2, 300, 128, 0, 0.1, None),
           VALUE, "q_scale inside o")
    # gradients
    b = [P + i * G for i in range(10)]
    expect(lib.attn_bwd_bf16(*b, 1, 2, 256, 64, 0, 0.125, None), HIP, "bwd valid")
    expect(lib.attn_bwd_bf16_gqa(*b, 2, 4, 2, 1000, 128, 1, 0.1, None), HIP, "bwd gqa valid")
    expect(lib.attn_bwd_bf16(*b[:9], b[8] + 64, 1, 2, 256, 64, 0, 0.125, None), VALUE, "ws in dv")
    expect(lib.attn_bwd_bf16(*b, 1, 2, 256, 256, 0, 0.125, None), SHAPE, "bwd d256")
    expect(lib.attn_bwd_bf16_workspace_bytes(2, 3, 100), 4800, "workspace bytes")
    expect(lib.attn_bwd_bf16_noalloc(*b[:9], 1, 2, 2, 256, 64, 0, 0.125, None), HIP, "noalloc valid")
    expect(lib.attn_bwd_bf16_noalloc(*b[:9], 1, 2, 2, (16 << 20) // 16 + 1, 64, 0, 0.125, None),
           SCRATCH, "noalloc too large")
    expect(lib.attn_bwd_bf16_noalloc(*b[:8], b[7] + 64, 1, 2, 2, 256, 64, 0, 0.125, None), VALUE,
           "noalloc dv in dk")
    # pre-passes
    q = [P + i * G for i in range(4)]
    expect(lib.blockquant_hadamard(*q, 2, 3, 300, 128, 128, None), HIP, "blockquant valid")
    expect(lib.blockquant_hadamard(*q, 2, 3, 300, 128, 0, None), HIP, "blockquant per-tensor")
    expect(lib.blockquant_hadamard(*q[:3], None, 2, 3, 300, 128, 128, None), HIP, "no signs")
    expect(lib.blockquant_hadamard(*q, 2, 3, 300, 128, 64, None), VALUE, "block_rows 64")
    expect(lib.blockquant_hadamard(q[0], q[1], q[2], q[2] + 4, 2, 3, 300, 128, 128, None), VALUE,
           "signs in scale")
    r = [P + i * G for i in range(6)]
    expect(lib.rope_blockquant_hadamard(*r, 1, 1, 2, 130, 64, 128, None), HIP, "rope valid")
    expect(lib.rope_blockquant_hadamard(*r, 2, 1, 2, 130, 64, 128, None), VALUE, "rope pairing 2")
    for code in range(-7, 1):
        expect(isinstance(lib.exattn_strerror(code), bytes), True, "strerror")
    expect(lib.exattn_abi_version(), 9, "abi version")
    print(f"ASAN_CHECKS_OK {checks}", flush=True)
''')


def test_abi_validation_under_address_sanitizer():
    assert os.path.exists(LIB), f"{LIB} missing: run __graft_entry__.build()"
    sys.path.insert(0, os.path.join(ROOT, "tests", "asan"))
    import build_host_asan
    env = dict(os.environ, LD_PRELOAD=build_host_asan.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=23")
    code = f"ROOT = {ROOT!r}\nLIB = {LIB!r}\n" + CHILD
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ASAN_CHECKS_OK" in out, out[-3000:]
    assert "AddressSanitizer" not in out, out[-3000:]
