// Reference outputs of PyTorch's CPU Philox4x32-10 engine (at::Philox4_32,
// header-only), used by the oracle's pin tests as an implementation of the
// generator independent of the oracle's own.
// stdin: lines "seed subsequence offset count"; stdout: count words per line.
#include <ATen/core/PhiloxRNGEngine.h>

#include <cinttypes>
#include <cstdio>

int main()
{
    unsigned long long seed, subseq, offset, count;
    while (std::scanf("%llu %llu %llu %llu", &seed, &subseq, &offset, &count) == 4) {
        at::Philox4_32 engine(seed, subseq, offset);
        for (unsigned long long i = 0; i < count; ++i)
            std::printf("%" PRIu32 "%c", engine(), i + 1 == count ? '\n' : ' ');
    }
    return 0;
}
