// Host check of the wave-structured transforms' output order (no GPU calls):
// for every supported length the map from storage position to frequency is a
// permutation, complementing the position complements the frequency (which
// the convolution's mirrored spectrum reads rely on), the compile-time and
// run-time forms of the map agree, and the root z = -1 (k = M/2) sits at
// position 512 (where the root-value kernels place its finite formula).
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "wfft.hpp"

using namespace ssm;

template <int LOGM>
static int check_static() {
    using G = WGeo<LOGM>;
    int bad = 0;
    for (int wave = 0; wave < G::W; ++wave)
        for (int e = 0; e < 16; ++e)
            for (int lane = 0; lane < 64; ++lane) {
                const int pos = (16 * wave + e) * 64 + lane;
                if (wf_freq<LOGM>(wave, e, lane) != wf_freq_rt(LOGM, pos)) ++bad;
            }
    return bad;
}

int main(int argc, char** argv) {
    if (argc == 3 && argv[1][0] == 'd') {  // "dump LOGM": the frequency at each position, one per line
        const int logm = atoi(argv[2]);
        if (logm < 10 || logm > 16) return 2;
        for (int pos = 0; pos < (1 << logm); ++pos) printf("%d\n", wf_freq_rt(logm, pos));
        return 0;
    }
    int bad = check_static<10>() + check_static<11>() + check_static<12>() + check_static<13>() + check_static<14>();
    if (bad) {
        printf("static and run-time maps differ at %d positions\n", bad);
        return 1;
    }
    for (int logm = 10; logm <= 16; ++logm) {
        const int M = 1 << logm;
        std::vector<char> seen(M, 0);
        int half_pos = -1;
        for (int pos = 0; pos < M; ++pos) {
            const int k = wf_freq_rt(logm, pos);
            if (k < 0 || k >= M || seen[k]) {
                printf("M = %d: position %d maps to %d (out of range or repeated)\n", M, pos, k);
                return 1;
            }
            seen[k] = 1;
            if (wf_freq_rt(logm, M - 1 - pos) != M - 1 - k) {
                printf("M = %d: complement of position %d is not the complement of %d\n", M, pos, k);
                return 1;
            }
            if (2 * k == M) half_pos = pos;
        }
        if (half_pos != 512) {
            printf("M = %d: k = M/2 at position %d, not 512\n", M, half_pos);
            return 1;
        }
    }
    printf("ok: positions 1024..65536\n");
    return 0;
}
