// ce_roundtrip — the C ABI used from plain host code, without Python or torch:
// reads a CE problem from a file, runs lmhead_loss_fwd and lmhead_loss_bwd
// (mean reduction, upstream gradient 1) on device 0 and writes the outputs.
//
// Input file (little-endian): int64 n, hidden, vocab, chunk; uint16 H[n*hidden]
// and W[vocab*hidden] (bf16 bits); int32 targets[n].
// Output file: float loss; float lse[n]; uint16 dH[n*hidden], dW[vocab*hidden];
// int32 device error code; int64 error row.
// Exit status: 0 ok, 1 usage or file error, 2 no usable device, 3 library or
// HIP error (the status string is printed).
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <vector>

#include "lmhead.h"

static int fail_hip(const char* what, hipError_t e) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 3;
}
static int fail_lib(const char* what, int st) {
    fprintf(stderr, "%s: %s (status %d)\n", what, lmhead_status_string(st), st);
    return 3;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s INPUT OUTPUT\n", argv[0]);
        return 1;
    }
    FILE* f = fopen(argv[1], "rb");
    if (!f) { perror(argv[1]); return 1; }
    int64_t dims[4];
    if (fread(dims, sizeof dims, 1, f) != 1) { fclose(f); fprintf(stderr, "short input\n"); return 1; }
    const int64_t n = dims[0], hidden = dims[1], vocab = dims[2], chunk = dims[3];
    if (n < 0 || hidden <= 0 || vocab <= 0 || chunk <= 0 || n > (1 << 20) || hidden > 65536 ||
        vocab > (1 << 24)) {
        fclose(f);
        fprintf(stderr, "implausible sizes\n");
        return 1;
    }
    std::vector<uint16_t> H((size_t)(n * hidden)), W((size_t)(vocab * hidden));
    std::vector<int32_t> t((size_t)n);
    const bool ok = fread(H.data(), 2, H.size(), f) == H.size() && fread(W.data(), 2, W.size(), f) == W.size() &&
                    fread(t.data(), 4, t.size(), f) == t.size();
    fclose(f);
    if (!ok) { fprintf(stderr, "short input\n"); return 1; }

    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        fprintf(stderr, "no HIP device\n");
        return 2;
    }
    hipError_t e = hipSetDevice(0);
    if (e != hipSuccess) return fail_hip("hipSetDevice", e);

    lmhead_problem p = {};
    p.n = n;
    p.hidden = hidden;
    p.vocab = vocab;
    p.chunk = chunk;
    p.num_valid = -1;
    p.k = 1;
    const size_t ws_bytes = lmhead_workspace_size(&p, LMHEAD_ENTRY_CE_MEAN, 1);
    if (ws_bytes == 0) { fprintf(stderr, "problem rejected by lmhead_workspace_size\n"); return 3; }

    void *dH_in = nullptr, *dW_in = nullptr, *d_t = nullptr, *d_loss = nullptr, *d_lse = nullptr,
         *d_grad = nullptr, *d_dH = nullptr, *d_dW = nullptr, *d_ws = nullptr;
    const size_t hb = H.size() * 2 + 16, wb = W.size() * 2 + 16;
    if ((e = hipMalloc(&dH_in, hb)) != hipSuccess || (e = hipMalloc(&dW_in, wb)) != hipSuccess ||
        (e = hipMalloc(&d_t, t.size() * 4 + 16)) != hipSuccess || (e = hipMalloc(&d_loss, 16)) != hipSuccess ||
        (e = hipMalloc(&d_lse, (size_t)n * 4 + 16)) != hipSuccess || (e = hipMalloc(&d_grad, 16)) != hipSuccess ||
        (e = hipMalloc(&d_dH, hb)) != hipSuccess || (e = hipMalloc(&d_dW, wb)) != hipSuccess ||
        (e = hipMalloc(&d_ws, ws_bytes)) != hipSuccess)
        return fail_hip("hipMalloc", e);
    const float one = 1.0f;
    if ((e = hipMemcpy(dH_in, H.data(), H.size() * 2, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(dW_in, W.data(), W.size() * 2, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(d_t, t.data(), t.size() * 4, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(d_grad, &one, 4, hipMemcpyHostToDevice)) != hipSuccess)
        return fail_hip("hipMemcpy", e);
    hipStream_t s;
    if ((e = hipStreamCreate(&s)) != hipSuccess) return fail_hip("hipStreamCreate", e);

    int st = lmhead_loss_fwd(&p, LMHEAD_ENTRY_CE_MEAN, dH_in, dW_in, (const int32_t*)d_t, (float*)d_loss,
                             (float*)d_lse, d_ws, ws_bytes, s);
    if (st != LMHEAD_OK) return fail_lib("lmhead_loss_fwd", st);
    st = lmhead_loss_bwd(&p, LMHEAD_ENTRY_CE_MEAN, dH_in, dW_in, (const int32_t*)d_t, nullptr,
                         (const float*)d_lse, nullptr, (const float*)d_grad, nullptr, d_dH, d_dW, d_ws,
                         ws_bytes, s);
    if (st != LMHEAD_OK) return fail_lib("lmhead_loss_bwd", st);
    int32_t code = 0;
    int64_t row = -1;
    st = lmhead_read_device_error(d_ws, s, &code, &row);   // synchronises the stream
    if (st != LMHEAD_OK) return fail_lib("lmhead_read_device_error", st);

    float loss = 0.0f;
    std::vector<float> lse((size_t)n);
    std::vector<uint16_t> gH(H.size()), gW(W.size());
    if ((e = hipMemcpy(&loss, d_loss, 4, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(lse.data(), d_lse, lse.size() * 4, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(gH.data(), d_dH, gH.size() * 2, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(gW.data(), d_dW, gW.size() * 2, hipMemcpyDeviceToHost)) != hipSuccess)
        return fail_hip("hipMemcpy back", e);
    (void)hipStreamDestroy(s);
    for (void* q : {dH_in, dW_in, d_t, d_loss, d_lse, d_grad, d_dH, d_dW, d_ws}) (void)hipFree(q);

    FILE* o = fopen(argv[2], "wb");
    if (!o) { perror(argv[2]); return 1; }
    const bool wok = fwrite(&loss, 4, 1, o) == 1 && fwrite(lse.data(), 4, lse.size(), o) == lse.size() &&
                     fwrite(gH.data(), 2, gH.size(), o) == gH.size() &&
                     fwrite(gW.data(), 2, gW.size(), o) == gW.size() && fwrite(&code, 4, 1, o) == 1 &&
                     fwrite(&row, 8, 1, o) == 1;
    fclose(o);
    if (!wok) { fprintf(stderr, "write failed\n"); return 1; }
    printf("ok: n=%lld vocab=%lld loss=%.6f error_code=%d\n", (long long)n, (long long)vocab, loss, code);
    return 0;
}
