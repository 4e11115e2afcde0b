"""Host-side validation calls of the C ABI, run by test_abi_sanitized.py in a
process that preloads the sanitizer runtime (no torch, no GPU: every call
here returns its status before any HIP call).  Usage:
python abi_sanitize_calls.py <path to a sanitized libgdn.so>."""

import ctypes
import sys

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_WS, ERR_HIP, ERR_SCRATCH, ERR_ALIAS = range(8)
P = ctypes.c_void_p(256)  # a fake, 16-byte aligned "device" pointer: never dereferenced
D = [ctypes.c_void_p((i + 1) << 40) for i in range(24)]  # distinct fake pointers, 1 TiB apart
N = None
SCRATCH_BYTES = 256 * 1024 * 1024


def main(path):
    # the sanitizer runtime is in the process (the instrumented library
    # would not load without it)
    assert hasattr(ctypes.CDLL(None), "__asan_init"), "the sanitizer runtime is not preloaded"
    lib = ctypes.CDLL(path)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "gdn_forward": ([i32] * 7 + [vp] * 8, ctypes.c_int),
        "gdn_forward_snapshots": ([i32] * 8 + [vp] * 9, ctypes.c_int),
        "gdn_rollback_select": ([i32] * 5 + [vp] * 4, ctypes.c_int),
        "gdn_forward_snapshots_after_rollback": ([i32] * 10 + [vp] * 11, ctypes.c_int),
        "gdn_prefill_workspace_size": ([i32] * 6, sz),
        "gdn_prefill_chunked": ([i32] * 6 + [vp] * 8 + [sz, vp], ctypes.c_int),
        "gdn_forward_qk_broadcast": ([i32] * 10 + [vp] * 9, ctypes.c_int),
        "gdn_prefill_chunked_qk_broadcast": ([i32] * 8 + [vp] * 8 + [sz, vp], ctypes.c_int),
        "gdn_prefill_chunked_snapshots": ([i32] * 9 + [vp] * 9 + [sz, vp], ctypes.c_int),
        "gdn_prefill_kda_workspace_size": ([i32] * 6, sz),
        "gdn_prefill_chunked_kda": ([i32] * 8 + [vp] * 8 + [sz, vp], ctypes.c_int),
        "gdn_prefill_workspace_size_ex": ([i32] * 8, sz),
        "gdn_prefill_chunked_ex": ([i32] * 11 + [vp] * 9 + [sz, vp], ctypes.c_int),
        "gdn_prefill_chunked_ex_after_rollback": ([i32] * 11 + [vp] * 10 + [sz, vp, vp], ctypes.c_int),
        "gdn_prefill_chunked_ex_noalloc": ([i32] * 11 + [vp] * 9, ctypes.c_int),
        "gdn_prefill_varlen_workspace_size": ([i32] * 6, sz),
        "gdn_prefill_chunked_varlen": ([i32] * 8 + [vp] * 9 + [sz, vp], ctypes.c_int),
        "gdn_prefill_varlen_workspace_size_ex": ([i32] * 8, sz),
        "gdn_prefill_chunked_varlen_ex": ([i32] * 10 + [vp] * 9 + [sz, vp], ctypes.c_int),
        "gdn_status_str": ([ctypes.c_int], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    checks = []

    def expect(got, want, what):
        checks.append((got == want, what, got, want))

    # token kernels
    fwd = lib.gdn_forward
    expect(fwd(1, 1, 1, 64, 64, 1, 0, N, P, P, P, P, P, P, N), ERR_NULL, "forward q NULL")
    expect(fwd(-1, 1, 1, 64, 64, 1, 0, P, P, P, P, P, P, P, N), ERR_SHAPE, "forward B < 0")
    expect(fwd(1, 1, 1, 96, 96, 1, 0, P, P, P, P, P, P, P, N), ERR_UNSUP, "forward d = 96")
    expect(fwd(1, 1, 1, 64, 64, 7, 0, P, P, P, P, P, P, P, N), ERR_UNSUP, "forward dtype")
    expect(fwd(1, 1, 1, 64, 64, 1, 0, ctypes.c_void_p(258), P, P, P, P, P, P, N), ERR_UNSUP, "forward align")
    expect(fwd(0, 1, 1, 64, 64, 1, 0, P, P, P, P, P, P, P, N), OK, "forward B = 0")
    expect(lib.gdn_forward_snapshots(1, 1, 1, 64, 64, 1, 0, 0, P, P, P, P, P, P, N, P, N), ERR_SHAPE, "K = 0")
    fb = lib.gdn_forward_qk_broadcast
    expect(fb(1, 1, 4, 3, 0, 64, 64, 1, 0, 1, P, P, P, P, P, P, N, P, N), ERR_SHAPE, "H_qk not dividing H")
    expect(fb(1, 1, 4, 2, 2, 64, 64, 1, 0, 1, P, P, P, P, P, P, N, P, N), ERR_UNSUP, "head map")
    rb = lib.gdn_rollback_select
    expect(rb(1, 1, 4, 64, 64, N, P, N, N), ERR_NULL, "rollback accepted NULL")
    expect(rb(1, 1, 4, 3, 3, P, P, N, N), ERR_UNSUP, "rollback odd tile")
    expect(rb(0, 1, 4, 64, 64, P, P, N, N), OK, "rollback B = 0")
    far = lib.gdn_forward_snapshots_after_rollback
    expect(far(1, 1, 1, 1, 0, 64, 64, 1, 0, 4, N, P, P, P, P, P, P, N, P, N, N), ERR_NULL, "fused accepted NULL")
    expect(far(1, 1, 4, 3, 0, 64, 64, 1, 0, 4, P, P, P, P, P, P, P, N, P, N, N), ERR_SHAPE, "fused H_qk")
    expect(far(0, 1, 1, 1, 0, 64, 64, 1, 0, 4, N, P, P, P, P, P, P, N, P, N, N), OK, "fused B = 0")
    # prefill entry points
    need = lib.gdn_prefill_workspace_size(1, 100, 2, 128, 128, 64)
    expect(need > 0, True, "workspace size")
    expect(lib.gdn_prefill_workspace_size(1, 100, 2, 128, 128, 32), 0, "workspace size chunk 32")
    pf = lib.gdn_prefill_chunked
    expect(pf(1, 100, 2, 128, 128, 64, N, P, P, P, P, P, P, P, need, N), ERR_NULL, "prefill q NULL")
    expect(pf(1, 100, 2, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], need - 1, N), ERR_WS, "prefill ws short")
    huge_T = (1 << 31) // (16 * 128 * 4)
    expect(pf(1, huge_T, 16, 128, 128, 64, P, P, P, P, P, P, P, P, 1 << 40, N), ERR_UNSUP, "prefill 2^31")
    par = lib.gdn_prefill_chunked_ex_after_rollback
    need_ex = lib.gdn_prefill_workspace_size_ex(1, 100, 2, 128, 128, 64, 1, 0)
    expect(par(1, 100, 2, 2, 0, 128, 128, 64, 1, 0, 4, N, P, P, P, P, P, P, N, P, P, need_ex, N, N), ERR_NULL,
           "prefill fused accepted NULL")
    expect(par(1, 100, 2, 2, 0, 128, 128, 64, 1, 0, 4, D[0], D[1], D[2], D[3], D[4], D[5], D[6], N, D[7], D[8], need_ex - 1, N, N), ERR_WS,
           "prefill fused ws short")
    expect(par(0, 100, 2, 2, 0, 128, 128, 64, 1, 0, 4, N, P, P, P, P, P, P, N, P, P, 0, N, N), OK,
           "prefill fused B = 0")
    kneed = lib.gdn_prefill_kda_workspace_size(1, 100, 4, 128, 128, 64)
    pk = lib.gdn_prefill_chunked_kda
    expect(pk(1, 100, 4, 4, 0, 128, 128, 64, P, P, P, ctypes.c_void_p(260), P, P, P, P, kneed, N),
           ERR_UNSUP, "kda gate alignment")
    ps = lib.gdn_prefill_chunked_snapshots
    expect(ps(2, 100, 4, 4, 0, 128, 128, 64, 4, P, P, P, P, P, N, P, P, P, need, N), ERR_NULL, "snapshots state")
    wsx = lib.gdn_prefill_workspace_size_ex
    pe = lib.gdn_prefill_chunked_ex
    expect(pe(1, 100, 4, 4, 0, 128, 128, 64, 5, 0, 1, P, P, P, P, P, P, N, P, P, 1 << 30, N), ERR_UNSUP, "ex dtype")
    kf = wsx(1, 100, 4, 128, 128, 64, 0, 1)
    expect(pe(1, 100, 4, 4, 0, 128, 128, 64, 0, 1, 1, D[0], D[1], D[2], D[3], D[4], D[5], N, D[6], D[7], kf - 1, N), ERR_WS, "ex ws short")
    pn = lib.gdn_prefill_chunked_ex_noalloc
    n = SCRATCH_BYTES // wsx(1, 64, 1, 128, 128, 64, 1, 0)
    expect(pn(1, 64 * n + 1, 1, 1, 0, 128, 128, 64, 1, 0, 1, D[0], D[1], D[2], D[3], D[4], D[5], N, D[6], N), ERR_SCRATCH,
           "noalloc beyond the scratch array")
    expect(pn(1, 0, 4, 4, 0, 128, 128, 64, 1, 0, 1, N, N, N, N, N, P, N, N, N), OK, "noalloc T = 0")
    vneed = lib.gdn_prefill_varlen_workspace_size(3, 300, 4, 128, 128, 64)
    pv = lib.gdn_prefill_chunked_varlen
    expect(pv(3, 300, 4, 2, 0, 128, 128, 64, N, P, P, P, P, P, P, P, P, vneed, N), ERR_NULL, "varlen cu NULL")
    expect(pv(3, 300, 4, 2, 0, 128, 128, 64, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], D[8], vneed - 1, N), ERR_WS, "varlen ws")
    vx = lib.gdn_prefill_varlen_workspace_size_ex(3, 300, 4, 128, 128, 64, 0, 1)
    pvx = lib.gdn_prefill_chunked_varlen_ex
    expect(pvx(3, 300, 4, 2, 0, 128, 128, 64, 0, 1, D[0], D[1], D[2], D[3], D[4], D[5], D[6], D[7], D[8], vx - 1, N), ERR_WS, "varlen ex ws")
    expect(pvx(3, 300, 4, 2, 0, 128, 128, 64, 0, 3, P, P, P, P, P, P, P, P, P, vx, N), ERR_UNSUP, "varlen ex gate")
    for s in list(range(8)) + [99]:
        expect(bool(lib.gdn_status_str(s)), True, f"status string {s}")
    bad = [c for c in checks if not c[0]]
    for _, what, got, want in bad:
        print(f"FAIL {what}: got {got}, want {want}")
    print(f"{len(checks) - len(bad)} of {len(checks)} checks ok")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
