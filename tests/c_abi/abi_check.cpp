// abi_check.cpp -- the library through its C ABI alone: no Python, no torch.
//
// Builds the four factorized layouts ("OpenAI Sparse Transformer",
// "Factorized Attention Patterns"), runs sa_fwd and sa_bwd on buffers from
// hipMalloc, and compares every output with the fp64 oracle (test
// infrastructure, linked only here) within the library's tolerances:
// O max-abs 2e-2, lse 1e-3 (non-empty rows; -inf on empty ones), dQ/dK/dV
// relative L2 5e-2.  Also checks that a bad call returns an error status
// with a message.  Exit status 0 when everything holds.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sa.h"

extern "C" {
void oracle_head_fwd(int pattern, int64_t l, int64_t c, int64_t n, int d, double scale, const double* q,
                     const double* k, const double* v, const int64_t* rows, int64_t nrows, double* o, double* lse);
void oracle_head_bwd(int pattern, int64_t l, int64_t c, int64_t n, int d, double scale, const double* q,
                     const double* k, const double* v, const double* dout, const int64_t* qrows, int64_t nq,
                     const int64_t* kcols, int64_t nk, double* dq, double* dk, double* dv, double* o_out,
                     double* lse_out);
}

namespace {

int failures = 0;

#define CHECK_HIP(x)                                                                   \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            return 2;                                                                  \
        }                                                                              \
    } while (0)

// splitmix64: a seeded stream of 64-bit words (input generation only).
uint64_t mix(uint64_t& s)
{
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

// Approximately standard normal: sum of four uniforms, centred and scaled.
double normalish(uint64_t& s)
{
    double t = 0.0;
    for (int a = 0; a < 4; ++a) t += (double)(mix(s) >> 11) * (1.0 / 9007199254740992.0);
    return (t - 2.0) * std::sqrt(3.0);
}

// float -> bf16 bits, round to nearest even; bf16 bits -> double exactly.
uint16_t to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
double from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
}

void expect(bool ok, const char* what, int h, double value, double bound)
{
    std::printf("%-4s head %d: %.3e (bound %.1e) %s\n", what, h, value, bound, ok ? "ok" : "FAIL");
    if (!ok) ++failures;
}

}  // namespace

int main()
{
    const int B = 1, H = 4, d = 64;
    const int64_t n = 512, l = 64, c = 16;
    const double scale = 0.125;
    const int pats[H] = {SA_STRIDED_A, SA_STRIDED_B, SA_FIXED_A, SA_FIXED_B};
    const size_t elems = (size_t)B * H * n * d, rows = (size_t)B * H * n;

    // Inputs: bf16 values of N(0,1)/sqrt(d) for q, k, v and N(0,1) for dO.
    std::vector<uint16_t> hq(elems), hk(elems), hv(elems), hdo(elems);
    uint64_t s = 20190423;
    for (size_t a = 0; a < elems; ++a) {
        hq[a] = to_bf16((float)(normalish(s) / 8.0));
        hk[a] = to_bf16((float)(normalish(s) / 8.0));
        hv[a] = to_bf16((float)(normalish(s) / 8.0));
        hdo[a] = to_bf16((float)normalish(s));
    }

    sa_layout_t* lay[H];
    for (int h = 0; h < H; ++h) {
        const int st = sa_layout_build(pats[h], n, l, pats[h] == SA_FIXED_B ? c : 1, 64, &lay[h]);
        if (st != SA_OK) {
            std::printf("sa_layout_build: %s\n", sa_last_error());
            return 2;
        }
    }

    void *q, *k, *v, *o, *dout, *dq, *dk, *dv, *ws;
    float* lse;
    const size_t bytes = elems * 2, ws_bytes = sa_bwd_workspace_size(B, H, n, d);
    CHECK_HIP(hipMalloc(&q, bytes));
    CHECK_HIP(hipMalloc(&k, bytes));
    CHECK_HIP(hipMalloc(&v, bytes));
    CHECK_HIP(hipMalloc(&o, bytes));
    CHECK_HIP(hipMalloc(&dout, bytes));
    CHECK_HIP(hipMalloc(&dq, bytes));
    CHECK_HIP(hipMalloc(&dk, bytes));
    CHECK_HIP(hipMalloc(&dv, bytes));
    CHECK_HIP(hipMalloc(&ws, ws_bytes));
    CHECK_HIP(hipMalloc((void**)&lse, rows * 4));
    CHECK_HIP(hipMemcpy(q, hq.data(), bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(k, hk.data(), bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(v, hv.data(), bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dout, hdo.data(), bytes, hipMemcpyHostToDevice));

    // A bad call: NULL output.  It must fail on the host with a message.
    int st = sa_fwd(lay, B, H, n, d, SA_BF16, (float)scale, q, k, v, nullptr, lse, nullptr);
    std::printf("sa_fwd(o = NULL) -> %d (%s): %s\n", st, sa_status_string(st), sa_last_error());
    if (st != SA_ERR_INVALID_ARG || std::strlen(sa_last_error()) == 0) ++failures;

    st = sa_fwd(lay, B, H, n, d, SA_BF16, (float)scale, q, k, v, o, lse, nullptr);
    if (st == SA_OK)
        st = sa_bwd(lay, B, H, n, d, SA_BF16, (float)scale, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, nullptr);
    if (st != SA_OK) {
        std::printf("call failed: %s\n", sa_last_error());
        return 2;
    }
    CHECK_HIP(hipDeviceSynchronize());
    std::vector<uint16_t> go(elems), gdq(elems), gdk(elems), gdv(elems);
    std::vector<float> glse(rows);
    CHECK_HIP(hipMemcpy(go.data(), o, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gdq.data(), dq, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gdk.data(), dk, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gdv.data(), dv, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(glse.data(), lse, rows * 4, hipMemcpyDeviceToHost));

    const size_t he = (size_t)n * d;
    std::vector<double> dq64(he), dk64(he), dv64(he), q64(he), k64(he), v64(he), do64(he), o64(he), lse64(n);
    for (int h = 0; h < H; ++h) {
        const size_t base = (size_t)h * he;
        for (size_t a = 0; a < he; ++a) {
            q64[a] = from_bf16(hq[base + a]);
            k64[a] = from_bf16(hk[base + a]);
            v64[a] = from_bf16(hv[base + a]);
            do64[a] = from_bf16(hdo[base + a]);
        }
        const int64_t cc = pats[h] == SA_FIXED_B ? c : 1;
        oracle_head_fwd(pats[h], l, cc, n, d, scale, q64.data(), k64.data(), v64.data(), nullptr, 0, o64.data(),
                        lse64.data());
        oracle_head_bwd(pats[h], l, cc, n, d, scale, q64.data(), k64.data(), v64.data(), do64.data(), nullptr, 0,
                        nullptr, 0, dq64.data(), dk64.data(), dv64.data(), nullptr, nullptr);
        double eo = 0.0, el = 0.0;
        bool inf_ok = true;
        for (size_t a = 0; a < he; ++a) eo = std::fmax(eo, std::fabs(from_bf16(go[base + a]) - o64[a]));
        for (int64_t i = 0; i < n; ++i) {
            const double g = glse[(size_t)h * n + i];
            if (std::isinf(lse64[i]))
                inf_ok = inf_ok && std::isinf(g) && g < 0;
            else
                el = std::fmax(el, std::fabs(g - lse64[i]));
        }
        expect(eo <= 2e-2, "O", h, eo, 2e-2);
        expect(el <= 1e-3 && inf_ok, "lse", h, el, 1e-3);
        const std::vector<uint16_t>* got[3] = {&gdq, &gdk, &gdv};
        const std::vector<double>* want[3] = {&dq64, &dk64, &dv64};
        const char* names[3] = {"dQ", "dK", "dV"};
        for (int t = 0; t < 3; ++t) {
            double num = 0.0, den = 0.0;
            for (size_t a = 0; a < he; ++a) {
                const double r = (*want[t])[a], e = from_bf16((*got[t])[base + a]) - r;
                num += e * e;
                den += r * r;
            }
            const double rel = std::sqrt(num / (den > 0 ? den : 1.0));
            expect(rel <= 5e-2, names[t], h, rel, 5e-2);
        }
    }
    for (int h = 0; h < H; ++h) sa_layout_destroy(lay[h]);
    void* bufs[] = {q, k, v, o, dout, dq, dk, dv, ws, lse};
    for (void* p : bufs) (void)hipFree(p);
    std::printf("%s\n", failures ? "FAILED" : "all checks passed");
    return failures ? 1 : 0;
}
