// Exercises the host side of libnaju.so -- argument checks, workspace and
// checkpoint sizing, error reporting -- for a build whose host code runs under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every call here returns
// before any device work: invalid arguments, empty problems (batch or d_inner
// 0), or the sizing functions.  Exit status 0 on success, 1 on an unexpected
// result.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "naju.h"

static int failures = 0;

static void expect(const char *what, naju_status_t got, naju_status_t want)
{
    const char *msg = naju_last_error();
    if (got != want) {
        std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want,
                     msg ? msg : "(null)");
        ++failures;
    }
    if (got != NAJU_OK && (!msg || std::strlen(msg) == 0)) {
        std::fprintf(stderr, "%s: no error message\n", what);
        ++failures;
    }
}

static naju_dims_t dims(int64_t Bt, int64_t L, int64_t Di, int64_t N, int io)
{
    naju_dims_t d;
    d.batch = Bt;
    d.seqlen = L;
    d.d_inner = Di;
    d.d_state = N;
    d.d_conv = 4;
    d.io = io;
    return d;
}

int main()
{
    alignas(256) static unsigned char buf[1 << 16];
    void *p = buf;                        // aligned stand-in for every tensor (never read)
    void *mis = buf + 2;                  // misaligned for fp32 and 256-byte workspaces
    float *fp = (float *)buf;
    const naju_op_t ops[] = {NAJU_OP_SCAN_FWD, NAJU_OP_SCAN_BWD, NAJU_OP_BLOCK_FWD,
                             NAJU_OP_BLOCK_BWD};

    // sizing over a range of shapes, including the largest accepted ones
    const int64_t Ls[] = {0, 1, 31, 32, 33, 127, 128, 129, 2048, 65536, (int64_t)1 << 30};
    const int64_t Dis[] = {0, 1, 8, 100, 1536, 4096, (int64_t)1 << 20};
    const int64_t Ns[] = {16, 64};
    for (int64_t L : Ls)
        for (int64_t Di : Dis)
            for (int64_t N : Ns)
                for (int io = 0; io < 2; ++io) {
                    naju_dims_t d = dims(2, L, Di, N, io);
                    for (naju_op_t op : ops) (void)naju_workspace_bytes(op, &d);
                    (void)naju_ckpt_bytes(&d);
                    if (io == NAJU_BF16 && Di % 8 == 0 && Di > 0)
                        (void)naju_mixer_workspace_bytes(&d, 768);
                }
    for (naju_op_t op : ops)
        if (naju_workspace_bytes(op, nullptr) != 0) {
            std::fprintf(stderr, "workspace bytes of NULL dims is not 0\n");
            ++failures;
        }

    naju_dims_t good = dims(2, 64, 32, 16, NAJU_BF16);
    const size_t ws_f = naju_workspace_bytes(NAJU_OP_SCAN_FWD, &good);
    // invalid dims
    expect("null dims", naju_scan_fwd(nullptr, p, p, p, p, p, fp, nullptr, p, nullptr, nullptr, p,
                                      ws_f, nullptr),
           NAJU_EINVAL);
    naju_dims_t bad = dims(-1, 64, 32, 16, NAJU_BF16);
    expect("negative batch", naju_scan_fwd(&bad, p, p, p, p, p, fp, nullptr, p, nullptr, nullptr,
                                           p, ws_f, nullptr),
           NAJU_EINVAL);
    bad = dims(2, 64, 32, 32, NAJU_BF16);
    expect("d_state 32", naju_scan_fwd(&bad, p, p, p, p, p, fp, nullptr, p, nullptr, nullptr, p,
                                       ws_f, nullptr),
           NAJU_EUNSUPPORTED);
    bad = dims(2, 64, 32, 16, 7);
    expect("io 7", naju_scan_fwd(&bad, p, p, p, p, p, fp, nullptr, p, nullptr, nullptr, p, ws_f,
                                 nullptr),
           NAJU_EINVAL);
    bad = dims(2, 64, 32, 16, NAJU_BF16);
    bad.d_conv = 3;
    expect("d_conv 3", naju_block_fwd(&bad, p, p, fp, nullptr, p, p, p, p, fp, nullptr, p,
                                      nullptr, nullptr, nullptr, p, 1 << 20, nullptr),
           NAJU_EUNSUPPORTED);
    bad = dims((int64_t)1 << 40, (int64_t)1 << 40, (int64_t)1 << 40, 16, NAJU_BF16);
    expect("huge", naju_scan_fwd(&bad, p, p, p, p, p, fp, nullptr, p, nullptr, nullptr, p, ws_f,
                                 nullptr),
           NAJU_EINVAL);
    // missing and misaligned tensors, workspace checks
    expect("null h", naju_scan_fwd(&good, nullptr, p, p, p, p, fp, nullptr, p, nullptr, nullptr,
                                   p, ws_f, nullptr),
           NAJU_EINVAL);
    expect("misaligned D", naju_scan_fwd(&good, p, p, p, p, p, (float *)mis, nullptr, p, nullptr,
                                         nullptr, p, ws_f, nullptr),
           NAJU_EINVAL);
    expect("misaligned x0", naju_scan_fwd(&good, p, p, p, p, p, fp, (float *)mis, p, nullptr,
                                          nullptr, p, ws_f, nullptr),
           NAJU_EINVAL);
    expect("null ws", naju_scan_fwd(&good, p, p, p, p, p, fp, nullptr, p, nullptr, nullptr,
                                    nullptr, ws_f, nullptr),
           NAJU_EWORKSPACE);
    expect("small ws", naju_scan_fwd(&good, p, p, p, p, p, fp, nullptr, p, nullptr, nullptr, p,
                                     ws_f - 1, nullptr),
           NAJU_EWORKSPACE);
    expect("misaligned ws", naju_scan_fwd(&good, p, p, p, p, p, fp, nullptr, p, nullptr, nullptr,
                                          mis, ws_f, nullptr),
           NAJU_EINVAL);
    const size_t ws_b = naju_workspace_bytes(NAJU_OP_BLOCK_BWD, &good);
    expect("block bwd null dz",
           naju_block_bwd(&good, p, p, fp, nullptr, p, p, p, p, fp, nullptr, nullptr, p, nullptr,
                          p, nullptr, fp, nullptr, p, p, p, p, fp, nullptr, p, ws_b, nullptr),
           NAJU_EINVAL);
    expect("block bwd small ws",
           naju_block_bwd(&good, p, p, fp, nullptr, p, p, p, p, fp, nullptr, nullptr, p, nullptr,
                          p, p, fp, nullptr, p, p, p, p, fp, nullptr, p, ws_b / 2, nullptr),
           NAJU_EWORKSPACE);
    const size_t ws_sb = naju_workspace_bytes(NAJU_OP_SCAN_BWD, &good);
    expect("scan bwd null dD",
           naju_scan_bwd(&good, p, p, p, p, p, fp, nullptr, nullptr, p, nullptr, p, p, p, p, p,
                         nullptr, nullptr, p, ws_sb, nullptr),
           NAJU_EINVAL);
    expect("step null x", naju_scan_step(&good, p, p, p, p, p, fp, nullptr, p, nullptr),
           NAJU_EINVAL);
    expect("block step null conv_state",
           naju_block_step(&good, p, p, fp, nullptr, p, p, p, p, fp, fp, p, nullptr), NAJU_EINVAL);
    naju_dims_t f32 = dims(2, 64, 32, 16, NAJU_F32);
    expect("mixer f32", naju_mixer_fwd(&f32, 64, p, nullptr, p, p, fp, nullptr, p, fp, p, fp, p,
                                       p, fp, p, p, p, 1 << 20, nullptr),
           NAJU_EUNSUPPORTED);
    expect("mixer d_model 12", naju_mixer_fwd(&good, 12, p, nullptr, p, p, fp, nullptr, p, fp, p,
                                              fp, p, p, fp, p, p, p, 1 << 20, nullptr),
           NAJU_EUNSUPPORTED);
    uint32_t flags = 0;
    expect("noalloc null y", naju_scan_fwd_noalloc(&good, p, p, p, p, p, fp, nullptr, nullptr,
                                                   nullptr, nullptr, &flags, nullptr),
           NAJU_EINVAL);
    // empty problems return before any device work
    naju_dims_t e0 = dims(0, 64, 32, 16, NAJU_BF16);
    expect("empty batch fwd", naju_scan_fwd(&e0, nullptr, nullptr, nullptr, nullptr, nullptr,
                                            nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                            0, nullptr),
           NAJU_OK);
    naju_dims_t e1 = dims(2, 64, 0, 16, NAJU_BF16);
    expect("empty width bwd",
           naju_block_bwd(&e1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, 0, nullptr),
           NAJU_OK);
    if (!naju_version() || std::strlen(naju_version()) == 0) ++failures;
    if (failures) return 1;
    std::printf("api driver: ok\n");
    return 0;
}
