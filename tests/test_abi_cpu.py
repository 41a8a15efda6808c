"""The C-ABI library without a GPU: it loads, exports what include/qknorm.h declares, and its
argument validation answers before any HIP call (no compute calls here)."""

import ctypes
import math
import os
import shutil
import subprocess

import pytest

from layerwise_qk_norm_amd import _lib

OK, NULL, SHAPE, DTYPE, EPS, ALIAS, ALIGN, HIPERR, SCRATCH = range(9)
F32, BF16 = 0, 1


def _gpu_present() -> bool:
    # Counting devices does not initialise HIP; validation tests hand the library fake device
    # addresses, which are only ever rejected, but they stay off machines with a GPU anyway.
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


no_gpu = pytest.mark.skipif(_gpu_present(), reason="fake-pointer validation runs on CPU only")


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _lib.header_entry_points()
    assert set(names) >= {"qknorm_fused", "qknorm_partial_sumsq", "qknorm_apply_with_stats",
                          "normproj_fold_weight", "normproj_deferred", "normproj_unfused",
                          "qkn_device_copy", "qkn_status_string", "qkn_last_hip_error",
                          "qknorm_shard_fused", "qknorm_shard_publish",
                          "normproj_fold_layernorm", "normproj_deferred_layernorm",
                          "normproj_layernorm_unfused", "qknorm_project_eliminated",
                          "normproj_deferred_layernorm_noalloc",
                          "qknorm_project_unfused"}
    for n in names:
        assert hasattr(L, n), n
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                             text=True).stdout
        exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
        assert set(names) <= exported
        # nothing but the C entry points is exported from the library's own code
        ours = {s for s in exported if s.startswith(("qkn", "qknorm", "normproj"))}
        assert ours == set(names)


def test_status_strings(L):
    for s in range(9):
        assert L.qkn_status_string(s) != b"unknown status"
    assert L.qkn_status_string(99) == b"unknown status"
    assert L.qkn_last_hip_error() == 0


# Fake, never-dereferenced device addresses (16-byte aligned, far apart).
A, B, C, D, G1, G2, E = (0x7F0000000000 + i * 0x10000000 for i in range(7))


def fused(L, T=4, eps=1e-6, dt=BF16, gdt=BF16, q=A, ldq=64, qo=B, ldqo=64, gq=G1, dq=64,
          k=C, ldk=64, ko=D, ldko=64, gk=G2, dk=64):
    return L.qknorm_fused(T, eps, dt, gdt, q, ldq, qo, ldqo, gq, dq, k, ldk, ko, ldko, gk, dk,
                          None)


@no_gpu
def test_fused_validation(L):
    assert fused(L, T=-1) == SHAPE
    assert fused(L, dt=7) == DTYPE
    assert fused(L, gdt=-1) == DTYPE
    assert fused(L, eps=float("nan")) == EPS
    assert fused(L, eps=-1.0) == EPS
    assert fused(L, eps=math.inf) == EPS
    assert fused(L, q=None) == NULL
    assert fused(L, qo=None) == NULL
    assert fused(L, gq=None) == NULL
    assert fused(L, gk=None) == NULL
    assert fused(L, dq=0) == SHAPE
    assert fused(L, ldq=32) == SHAPE          # ld < d
    assert fused(L, ldko=10) == SHAPE
    # T == 0 is a no-op whatever the pointers
    assert fused(L, T=0, q=None, qo=None, gq=None, k=None, ko=None, gk=None) == OK
    assert fused(L, q=A + 1) == ALIGN           # bf16 elements off their 2-byte alignment
    assert fused(L, ko=C + 1) == ALIGN
    assert fused(L, gdt=F32, gq=G1 + 2) == ALIGN  # fp32 gamma off 4 bytes
    assert fused(L, q=A + 2, qo=B + 2) == HIPERR  # element-aligned: accepted
    # partial overlap of q_out with q (shifted by one row) is rejected; so is K's output
    # landing on Q's input, or Q's output on a gamma
    assert fused(L, qo=A + 128) == ALIAS
    assert fused(L, ko=A) == ALIAS
    assert fused(L, qo=G1) == ALIAS
    assert fused(L, qo=A, ldqo=128, ldq=64) == ALIAS     # same base, different stride
    # Q and K as the two column blocks of one [T, 128] matrix, normalised in place: the blocks
    # interleave row by row but never share a byte
    blk = dict(q=A, ldq=128, qo=A, ldqo=128, k=A + 128, ldk=128, ko=A + 128, ldko=128)
    assert fused(L, **blk) == HIPERR           # accepted; the launch then finds no device
    # ... while a K block starting one column early runs into Q's last column
    assert fused(L, **dict(blk, k=A + 126, ko=A + 126)) == ALIAS
    # and blocks of different strides are compared by their hulls
    assert fused(L, **dict(blk, ldk=136, ldko=136)) == ALIAS


@no_gpu
def test_partial_and_apply_validation(L):
    P = L.qknorm_partial_sumsq
    assert P(-1, BF16, A, 64, 64, B, C, 64, 64, D, None) == SHAPE
    assert P(4, 5, A, 64, 64, B, C, 64, 64, D, None) == DTYPE
    assert P(4, BF16, A, 64, 64, None, C, 64, 64, D, None) == NULL
    assert P(4, BF16, A, 64, 65, B, C, 64, 64, D, None) == SHAPE
    assert P(4, BF16, A, 64, 64, A, C, 64, 64, D, None) == ALIAS   # psq on top of q
    assert P(4, BF16, A, 64, 64, B, C, 64, 64, B + 4, None) == ALIAS
    assert P(0, BF16, None, 1, 1, None, None, 0, 0, None, None) == OK
    assert P(4, BF16, A + 1, 64, 64, B, C, 64, 64, D, None) == ALIGN   # odd bf16 address
    assert P(4, BF16, A, 64, 64, B + 2, C, 64, 64, D, None) == ALIGN   # partials off 4 bytes

    def apply(T=4, eps=1e-6, n_ext=7, q=A, ldq=64, qo=B, ldqo=64, gq=G1, dl=64, df=512, pq=D,
              eq=D + 0x1000, lde=4):
        return L.qknorm_apply_with_stats(T, eps, BF16, BF16, n_ext, q, ldq, qo, ldqo, gq, dl, df,
                                         pq, eq, lde, None, 0, None, 0, None, 0, 0, None, None, 0,
                                         None)

    assert apply(n_ext=-1) == SHAPE
    assert apply(df=32) == SHAPE               # d_full < d_local
    assert apply(lde=3) == SHAPE               # ld_ext < T
    assert apply(eq=None) == NULL
    assert apply(pq=None) == NULL
    assert apply(eps=float("inf")) == EPS
    assert apply(qo=D) == ALIAS                # output over the own partials
    assert apply(qo=D + 0x1000 - 64) == ALIAS  # output running into ext
    assert apply(pq=D + 2) == ALIGN            # fp32 partials off 4 bytes
    assert apply(eq=D + 0x1000 + 2) == ALIGN


@no_gpu
def test_normproj_validation(L):
    F = L.normproj_fold_weight
    assert F(16, 16, F32, BF16, A, 16, G1, B, 16, None) == DTYPE
    assert F(16, 16, BF16, BF16, A, 8, G1, B, 16, None) == SHAPE      # ldw < N
    assert F(16, 16, BF16, BF16, A, 16, G1, B, 8, None) == SHAPE      # ldw_fold < N
    # W' is written [K, N] like W: any alignment and stride, in place allowed
    assert F(16, 16, BF16, BF16, A, 16, G1, B + 2, 17, None) == HIPERR
    assert F(16, 16, BF16, BF16, A, 16, G1, A, 16, None) == HIPERR
    assert F(16, 16, BF16, BF16, A, 16, G1, A + 32, 16, None) == ALIAS  # shifted overlap
    assert F(16, 16, BF16, BF16, A, 16, G1, A, 24, None) == ALIAS       # same base, other ld
    assert F(16, 16, BF16, BF16, A, 16, G1, G1 - 32, 16, None) == ALIAS
    assert F(16, 16, BF16, BF16, None, 16, G1, B, 16, None) == NULL
    P = L.normproj_deferred
    assert P(4, 16, 16, 1e-6, F32, A, 16, B, 16, C, 16, None) == DTYPE
    # w_fold is [K, N]: its stride covers N, not K
    assert P(4, 16, 24, 1e-6, BF16, A, 16, B, 16, C, 24, None) == SHAPE   # ldw < N
    assert P(4, 16, 8, 1e-6, BF16, A, 16, B, 8, C, 8, None) == HIPERR    # ldw < K is fine
    # any K, stride and 2-byte alignment runs (an element-load kernel where 16 bytes do not)
    assert P(4, 12, 16, 1e-6, BF16, A, 12, B, 16, C, 16, None) == HIPERR  # K % 8
    assert P(4, 1001, 16, 1e-6, BF16, A + 2, 1003, B + 2, 17, C + 2, 19, None) == HIPERR
    assert P(4, 16, 16, 1e-6, BF16, A + 1, 16, B, 16, C, 16, None) == ALIGN  # odd address
    assert P(4, 16, 16, 1e-6, BF16, A, 16, B + 1, 16, C, 16, None) == ALIGN
    assert P(4, 16, 16, 1e-6, BF16, A, 16, B, 16, C + 1, 16, None) == ALIGN
    assert P(4, 16, 64, 1e-6, BF16, A, 16, B, 64, B + 1024, 64, None) == ALIAS  # y on W' row 8
    assert P(4, 16, 64, 1e-6, BF16, A, 16, B, 64, B + 2048, 64, None) == HIPERR  # just past W'
    assert P(4, 16, 16, 1e-6, BF16, A, 16, B, 16, A + 32, 16, None) == ALIAS
    assert P(4, 16, 16, -1.0, BF16, A, 16, B, 16, C, 16, None) == EPS
    assert P(4, 16, 16, 1e-6, BF16, A, 16, B, 16, None, 16, None) == NULL
    assert P(0, 16, 16, 1e-6, BF16, None, 16, None, 16, None, 16, None) == OK
    U = L.normproj_unfused
    assert U(4, 16, 16, 1e-6, BF16, BF16, A, 16, G1, B, 16, A, 16, C, 16, None) == ALIAS
    assert U(4, 16, 16, 1e-6, BF16, BF16, A, 16, G1, B, 16, None, 16, C, 16, None) == NULL
    assert U(4, 16, 16, 1e-6, BF16, 9, A, 16, G1, B, 16, D, 16, C, 16, None) == DTYPE
    assert U(4, 16, 16, 1e-6, BF16, BF16, A, 16, G1, B, 16, D, 16, G1 - 32, 16, None) == ALIAS
    assert L.qkn_device_copy(A, A + 8, 64, None) == ALIAS
    assert L.qkn_device_copy(A, B, -1, None) == SHAPE
    assert L.qkn_device_copy(None, B, 0, None) == OK


@no_gpu
def test_layernorm_projection_validation(L):
    F = L.normproj_fold_layernorm
    assert F(16, 16, F32, BF16, A, 16, G1, G2, B, 16, C, D, None) == DTYPE
    assert F(16, 16, BF16, BF16, A, 8, G1, G2, B, 16, C, D, None) == SHAPE     # ldw < N
    assert F(16, 16, BF16, BF16, A, 16, G1, G2, B + 2, 16, C, D, None) == HIPERR
    assert F(16, 16, BF16, BF16, A, 16, G1, G2, B, 16, None, D, None) == NULL  # colsum needed
    assert F(16, 16, BF16, BF16, A, 16, G1, G2, B, 16, A, D, None) == ALIAS    # colsum on W
    assert F(16, 16, BF16, BF16, A, 16, G1, G2, B, 16, C, C + 32, None) == ALIAS
    assert F(16, 16, BF16, BF16, A, 16, G1, G2, B, 16, C, G2, None) == ALIAS   # bias on beta
    assert F(0, 16, BF16, BF16, None, 16, None, None, None, 16, None, None, None) == OK
    P = L.normproj_deferred_layernorm
    assert P(4, 16, 16, 1e-5, F32, A, 16, B, 16, C, D, G1, 16, None, None) == DTYPE
    assert P(4, 12, 16, 1e-5, BF16, A, 12, B, 16, C, D, G1, 16, None, None) == HIPERR  # K % 8
    assert P(4, 12, 16, 1e-5, BF16, A, 12, B, 12, C, D, G1, 16, None, None) == SHAPE  # ldw < N
    assert P(4, 16, 16, -1.0, BF16, A, 16, B, 16, C, D, G1, 16, None, None) == EPS
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, None, D, G1, 16, None, None) == NULL
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, C, 16, None, None) == ALIAS  # y on colsum
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, D, 16, None, None) == ALIAS  # y on bias
    # the row-statistics workspace: clear of every other operand (one that is not 8-byte
    # aligned is accepted and left unused)
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, G1, 16, E + 4, None) == HIPERR
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, G1, 16, G1 + 8, None) == ALIAS  # on y
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, G1, 16, A + 64, None) == ALIAS  # on x
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, G1, 16, B, None) == ALIAS      # on W'
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, G1, 16, C + 16, None) == ALIAS  # colsum
    assert P(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, G1, 16, D, None) == ALIAS      # bias
    assert P(0, 16, 16, 1e-5, BF16, None, 16, None, 16, None, None, None, 16, None, None) == OK
    # the variant with the library's static workspace: the same checks, then its size limit
    # (131072 rows) before any HIP call; within it, the lookup of the workspace finds no device
    S = L.normproj_deferred_layernorm_noalloc
    assert S(4, 16, 16, 1e-5, F32, A, 16, B, 16, C, D, G1, 16, None) == DTYPE
    assert S(4, 16, 16, -1.0, BF16, A, 16, B, 16, C, D, G1, 16, None) == EPS
    assert S(4, 16, 16, 1e-5, BF16, A, 16, B, 16, None, D, G1, 16, None) == NULL
    assert S(4, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, C, 16, None) == ALIAS
    assert S(0, 16, 16, 1e-5, BF16, None, 16, None, 16, None, None, None, 16, None) == OK
    assert S(131073, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, G1, 16, None) == SCRATCH
    assert S(131072, 16, 16, 1e-5, BF16, A, 16, B, 16, C, D, G1, 16, None) == HIPERR
    U = L.normproj_layernorm_unfused
    assert U(4, 16, 16, 1e-5, BF16, BF16, A, 16, G1, G2, B, 16, A, 16, C, 16, None) == ALIAS
    assert U(4, 16, 16, 1e-5, BF16, BF16, A, 16, G1, G2, B, 16, None, 16, C, 16, None) == NULL
    assert U(4, 16, 16, 1e-5, BF16, BF16, A, 16, G1 + 2, G2, B, 16, D, 16, C, 16, None) == HIPERR
    assert U(4, 16, 16, 1e-5, BF16, BF16, A, 16, G1 + 1, G2, B, 16, D, 16, C, 16, None) == ALIGN
    assert U(4, 16, 16, 1e-5, BF16, F32, A, 16, G1 + 2, G2, B, 16, D, 16, C, 16, None) == ALIGN
    assert U(4, 16, 16, 1e-5, BF16, 9, A, 16, G1, G2, B, 16, D, 16, C, 16, None) == DTYPE
    assert U(4, 16, 16, 1e-5, BF16, BF16, A, 16, G1, G2, B, 16, D, 16, G1 - 32, 16, None) == ALIAS
    assert U(4, 16, 16, 1e-5, BF16, BF16, A, 16, G1, G2, B, 16, D, 16, G2 - 32, 16, None) == ALIAS


@no_gpu
def test_project_eliminated_validation(L):
    def E(T=4, K=16, nq=8, nk=8, e2=1e-6, e1=1e-6, exact=0, gdt=BF16, x=A, ldx=16, w=B, ldw=16,
          gq=G1, gk=G2, y=C, ldy=16):
        return L.qknorm_project_eliminated(T, K, nq, nk, e2, e1, exact, gdt, x, ldx, w, ldw, gq,
                                           gk, y, ldy, None)

    assert E(nq=0) == SHAPE
    assert E(nk=-1) == SHAPE
    assert E(exact=2) == SHAPE
    assert E(ldy=15) == SHAPE                  # ldy < nq + nk
    assert E(e2=float("nan")) == EPS
    assert E(e1=-1.0) == EPS
    assert E(gdt=3) == DTYPE
    assert E(K=12, ldx=12) == HIPERR            # any K
    assert E(ldw=15) == SHAPE                   # ldw < nq + nk
    assert E(x=A + 1) == ALIGN
    assert E(gq=None) == NULL
    assert E(gk=None) == NULL
    assert E(y=A) == ALIAS                     # output over x
    assert E(y=G1 - 32) == ALIAS               # output running into gamma_q
    assert E(T=0, x=None, w=None, gq=None, gk=None, y=None) == OK


@no_gpu
def test_project_unfused_validation(L):
    def U(T=4, K=16, nq=8, nk=8, e2=1e-6, e1=1e-6, gdt=BF16, x=A, ldx=16, g1=G1, w=B, ldw=16,
          gq=G2, gk=G2 + 64, xn=D, ldxn=16, y=C, ldy=16):
        return L.qknorm_project_unfused(T, K, nq, nk, e2, e1, gdt, x, ldx, g1, w, ldw, gq, gk,
                                        xn, ldxn, y, ldy, None)

    assert U(nq=0) == SHAPE
    assert U(nk=-1) == SHAPE
    assert U(ldy=15) == SHAPE                  # ldy < nq + nk
    assert U(ldxn=8) == SHAPE                  # ldxn < K
    assert U(e2=float("nan")) == EPS
    assert U(e1=-1.0) == EPS
    assert U(gdt=3) == DTYPE
    assert U(K=12, ldx=12, ldxn=12) == HIPERR   # any K
    assert U(xn=D + 2) == HIPERR
    assert U(xn=D + 1) == ALIGN
    assert U(gq=None) == NULL
    assert U(gk=None) == NULL
    assert U(g1=None) == NULL
    assert U(xn=None) == NULL
    assert U(y=A) == ALIAS                     # output over x
    assert U(y=G2 - 32) == ALIAS               # output running into gamma_q
    assert U(xn=A) == ALIAS                    # scratch over x
    assert U(xn=G2 - 32) == ALIAS              # scratch running into gamma_q
    assert U(y=G1 - 32) == ALIAS               # output running into the pre-norm's gamma
    assert U(T=0, x=None, w=None, g1=None, gq=None, gk=None, xn=None, y=None) == OK


@no_gpu
def test_shard_validation(L):
    def shard(T=64, eps=1e-6, dt=BF16, n_ext=7, q=A, ldq=512, qo=B, dl=512, df=4096, psq=D,
              mail=D + 0x10000, ldm=64, epoch=1, pers=1, spin=100, to=G2 + 0x20000):
        return L.qknorm_shard_fused(T, eps, dt, BF16, n_ext, q, ldq, qo, ldq, G1, dl, df, psq,
                                    mail, ldm, None, 0, None, 0, None, 0, 0, None, None, 0,
                                    epoch, pers, spin, to, None)

    assert shard(n_ext=65) == SHAPE
    assert shard(n_ext=-1) == SHAPE
    assert shard(spin=-1) == SHAPE
    assert shard(pers=2) == SHAPE
    assert shard(dl=4096, ldq=4096) == SHAPE       # slice wider than 2048 bf16
    assert shard(df=256) == SHAPE                  # d_full < d_local
    assert shard(ldm=63) == SHAPE                  # mailbox stride < T
    assert shard(q=A + 1) == ALIGN                 # bf16 elements off their 2-byte alignment
    assert shard(q=A + 2, ldq=515) == HIPERR       # any element-aligned slice is accepted
    assert shard(dl=500, ldq=512) == HIPERR        # (element accesses; no device here)
    assert shard(mail=D + 0x10004) == ALIGN        # mailbox words not 8-byte aligned
    assert shard(psq=D + 4) == ALIGN
    assert shard(to=None) == NULL                  # waiting needs a timeout flag
    assert shard(mail=None) == NULL
    assert shard(qo=D) == ALIAS                    # output over the own partials
    assert shard(psq=D + 0x10000 + 64) == ALIAS    # own partials over the mailbox
    assert shard(to=D + 0x10000) == ALIAS          # timeout flag over the mailbox
    assert shard(T=0, q=None, qo=None, psq=None, mail=None, to=None) == OK
    # epoch 0 (complete mailbox): no timeout flag needed; the own partials are optional
    assert shard(epoch=0, to=None, psq=None) == HIPERR   # accepted; no device to launch on
    P = L.qknorm_shard_publish
    assert P(64, 7, A, 64, B, 63, None, 0, None, 0, 1, None) == SHAPE      # ld_mail < T
    assert P(-1, 7, A, 64, B, 64, None, 0, None, 0, 1, None) == SHAPE
    assert P(64, 7, A, 64, B + 4, 64, None, 0, None, 0, 1, None) == ALIGN
    assert P(64, 7, A, 64, A + 64, 64, None, 0, None, 0, 1, None) == ALIAS
    assert P(64, 7, A, 64, None, 64, None, 0, None, 0, 1, None) == NULL
    assert P(0, 7, None, 0, None, 0, None, 0, None, 0, 1, None) == OK


@no_gpu
def test_oversized_extents_are_rejected(L):
    """Sizes whose byte extent ((rows - 1) * ld + cols elements) passes 2^56 bytes, products
    that overflow 64 bits included, are QKN_ERR_SHAPE before any other check can wrap."""
    big = 1 << 40
    assert fused(L, T=big, ldq=big) == SHAPE
    assert fused(L, T=1 << 62, ldq=1 << 62) == SHAPE            # (T - 1) * ld overflows int64
    assert fused(L, T=big, ldk=big, ldko=big) == SHAPE
    # the bound itself: bf16 rows are sized as 4-byte elements, 2^54 elements in all
    edge = (1 << 54) - 64
    assert fused(L, T=2, ldq=edge, ldqo=64) != SHAPE          # exactly 2^56 bytes: accepted
    assert fused(L, T=2, ldq=edge + 1, ldqo=64) == SHAPE
    assert L.qknorm_partial_sumsq(big, BF16, A, big, 64, D, None, 0, 0, None, None) == SHAPE
    assert L.qknorm_apply_with_stats(4, 1e-6, BF16, BF16, big, A, 64, B, 64, G1, 64, 512, D,
                                     E, big, None, 0, None, 0, None, 0, 0, None, None, 0,
                                     None) == SHAPE            # ext [n_ext, ld_ext] too large
    assert L.qknorm_shard_fused(64, 1e-6, BF16, BF16, 7, A, 512, B, 512, G1, 512, 4096, D,
                                E, 1 << 62, None, 0, None, 0, None, 0, 0, None, None, 0, 1, 1,
                                100, G2, None) == SHAPE        # mailbox stride overflows
    assert L.qknorm_shard_publish(64, big, A, big, B, 64, None, 0, None, 0, 1, None) == SHAPE
    assert L.normproj_fold_weight(big, 64, BF16, BF16, A, big, G1, B, 64, None) == SHAPE
    assert L.normproj_fold_layernorm(big, 64, BF16, BF16, A, 64, G1, G2, B, big, D, E,
                                     None) == SHAPE
    assert L.normproj_deferred(big, 64, 64, 1e-6, BF16, A, big, B, 64, C, 64, None) == SHAPE
    assert L.normproj_deferred(4, 64, 64, 1e-6, BF16, A, 64, B, 64, C, 1 << 62, None) == SHAPE
    assert L.normproj_unfused(4, 64, 64, 1e-6, BF16, BF16, A, 64, G1, B, 64, D, 1 << 62, C, 64,
                              None) == SHAPE                   # the normalised-x workspace
    assert L.qknorm_project_eliminated(4, 16, 1 << 62, 1 << 62, 1e-6, 1e-6, 0, BF16, A, 16, B,
                                       16, G1, G2, C, 16, None) == SHAPE   # nq + nk overflows
    assert L.qkn_device_copy(A, B, (1 << 56) + 1, None) == SHAPE


def test_library_has_gfx950_code_object():
    """The shared object embeds a gfx950 offload bundle (checked on the file's bytes for the
    target id the build embeds)."""
    data = open(_lib.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_python_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    import layerwise_qk_norm_amd as q

    x = torch.zeros((2, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        q.qknorm_fused(x, torch.ones(8, dtype=torch.bfloat16))


def test_python_binding_refuses_strided_or_short_vectors():
    """Vectors travel as bare pointers: a strided view or a short tensor would be misread."""
    torch = pytest.importorskip("torch")
    _lib._vec(None, 8, "gamma")
    _lib._vec(torch.zeros(8), 8, "gamma")
    with pytest.raises(ValueError):
        _lib._vec(torch.zeros(16)[::2], 8, "gamma")
    with pytest.raises(ValueError):
        _lib._vec(torch.zeros(7), 8, "gamma")


def test_python_binding_refuses_undersized_matrices():
    """2-D operands are addressed from pointer and row stride: too few rows or columns would
    be read or written past the end of the buffer."""
    torch = pytest.importorskip("torch")
    _lib._mat(None, 4, 4, "y")
    _lib._mat(torch.zeros(4, 8), 4, 8, "y")
    for bad in (torch.zeros(3, 8), torch.zeros(4, 7), torch.zeros(32)):
        with pytest.raises(ValueError):
            _lib._mat(bad, 4, 8, "y")


def test_python_binding_row_strides():
    """Row strides come from the tensor; an empty tensor (numpy gives it zero strides) gets its
    width, and a view whose columns are not adjacent is refused."""
    torch = pytest.importorskip("torch")
    import numpy as np

    assert _lib._ld(torch.zeros(4, 8)) == 8
    assert _lib._ld(torch.zeros(4, 16)[:, 3:11]) == 16
    assert _lib._ld(torch.zeros(1, 8)) == 8
    empty = torch.from_numpy(np.zeros((0, 1001), np.float32))
    assert empty.stride() == (0, 0)
    assert _lib._ld(empty) == 1001
    assert _lib._ld(torch.zeros(5, 0)) == 1
    with pytest.raises(ValueError):
        _lib._ld(torch.zeros(4, 16)[:, ::2])
    with pytest.raises(ValueError):
        _lib._ld(torch.zeros(8))


def test_python_binding_copy_checks_sizes(monkeypatch):
    """The copy's byte count is checked against both tensors before the library is reached."""
    torch = pytest.importorskip("torch")
    monkeypatch.setattr(_lib, "_check_device", lambda *ts: None)
    reached = []
    monkeypatch.setattr(_lib, "lib", lambda: reached.append(1))
    u8 = torch.uint8
    for dst, src in ((torch.zeros(4, dtype=u8), torch.zeros(8, dtype=u8)),
                     (torch.zeros(8, dtype=u8), torch.zeros(4, dtype=u8)),
                     (torch.zeros(16, dtype=u8)[::2], torch.zeros(8, dtype=u8))):
        with pytest.raises(ValueError):
            _lib.qkn_device_copy(dst, src, 8)
    assert not reached


def test_python_binding_refuses_mismatched_dtypes():
    """One dtype code travels per group of operands: a companion of another dtype is refused."""
    torch = pytest.importorskip("torch")
    _lib._dtypes(torch.bfloat16, "w_fold", None, torch.zeros(2, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        _lib._dtypes(torch.bfloat16, "w_fold", torch.zeros(2, dtype=torch.float32))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.lib()
