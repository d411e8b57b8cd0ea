// Host-code check of the library's codebook derivation, built with the
// address and undefined-behaviour sanitizers by tests/test_host_sanitized.py.
// For every subspace width 2..64 and both readings it asks for the 8-level
// tables and checks that they are ordered and inside (0, 1); it also checks
// that invalid arguments are rejected.  Exit code 0 = every check passed.
#include <cmath>
#include <cstdio>

#include "pariskv.h"

int main() {
    int bad = 0;
    for (int kind = 0; kind < 2; ++kind) {
        for (int m = 2; m <= 64; ++m) {
            float lv[8], th[7];
            const pk_status st = kind == 0 ? pk_codebook(m, 8, lv, th) : pk_codebook_quantile(m, 8, lv, th);
            if (st != PK_OK) {
                std::printf("m=%d kind=%d: status %d\n", m, kind, (int)st);
                ++bad;
                continue;
            }
            for (int i = 0; i < 8; ++i) {
                const bool ok = std::isfinite(lv[i]) && lv[i] > 0.0f && lv[i] < 1.0f &&
                                (i == 0 || lv[i] > lv[i - 1]) &&
                                (i == 7 || (th[i] > lv[i] * lv[i] && th[i] < lv[i + 1] * lv[i + 1]));
                if (!ok) {
                    std::printf("m=%d kind=%d: entry %d out of order or range\n", m, kind, i);
                    ++bad;
                }
            }
        }
    }
    float lv[8], th[7];
    if (pk_codebook(1, 8, lv, th) != PK_ERR_INVALID) ++bad;
    if (pk_codebook(8, 4, lv, th) != PK_ERR_INVALID) ++bad;
    if (pk_codebook(8, 8, nullptr, th) != PK_ERR_INVALID) ++bad;
    if (pk_codebook_quantile(8, 8, lv, nullptr) != PK_ERR_INVALID) ++bad;
    std::printf("%s\n", bad == 0 ? "codebook host checks passed" : "codebook host checks FAILED");
    return bad == 0 ? 0 : 1;
}
